// Expert construction: the low-rank factors of the shared and routed experts.
//
// MCISLAB DeepRead summary of "Quant Experts", section "Method" (Shared Expert, Routed
// Experts): the layer's quantization error E = W_f - W_q is reconstructed by a low-rank shared
// expert, and the error left after it by one low-rank routed expert per cluster of
// token-dependent channels.  PaperDaily post "西交大提出Quant Experts：token级量化补偿",
// section "核心设计": the decomposition is a whitening SVD, which balances the scales of the
// directions before the SVD.  Here the whitening is diagonal (input channel j weighted by the
// RMS c_j of its calibration activations), and the truncated SVD of M = diag(w) E^T is the
// randomized subspace iteration of Halko, Martinsson and Tropp, "Finding structure with
// randomness" (SIAM Review 2011), Algorithms 4.4 and 5.1, with the Gaussian test matrix an
// input:
//   Y = M omega, Q = qr(Y); power_iters times: Q~ = qr(M^T Q), Q = qr(M Q~);
//   Z = M^T Q (= B^T with B = Q^T M);  B B^T = Z^T Z = U~ S^2 U~^T;  U = Q U~, V = Z U~ S^-1;
//   A = diag(1/w) U_r S_r^(1/2) (rows with w = 0 are zero), B = S_r^(1/2) V_r^T.
//
// The passes over E (d_out x d_in float32, up to ~1 GB for the largest linears) run on the
// GPU: the thin products M X and M^T X with X of k <= 128 columns (float32 FMAs, LDS tiles,
// contraction split over workgroups with atomic adds).  The host does the work on the thin
// matrices in double: Householder QR (Golub and Van Loan, "Matrix Computations", section
// 5.2.1) and the k x k symmetric eigenproblem.

#include <algorithm>
#include <cmath>
#include <thread>
#include <vector>

#include "qe_calib.h"
#include "qe_internal.h"
#include "qe_lowrank.h"

namespace qe {

namespace {

// ---------------------------------------------------------------- quantization error
// One workgroup per output channel: the row maximum of |W_f * s|, s_w = max / qmax, then
// the codes exactly as the weight quantizer takes them (float32, ties to even, clamp) and
// E = W_f - s_w * code / s.
__global__ __launch_bounds__(256) void quant_error_kernel(const float* __restrict__ W, const float* __restrict__ s,
                                                          int d_in, float qmax, float* __restrict__ E) {
    __shared__ float red[256];
    const float* row = W + (size_t)blockIdx.x * d_in;
    float* out = E + (size_t)blockIdx.x * d_in;
    const int tid = threadIdx.x;
    float amax = 0.0f;
    for (int j = tid; j < d_in; j += 256) amax = fmaxf(amax, fabsf(s ? row[j] * s[j] : row[j]));
    red[tid] = amax;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if (tid < h) red[tid] = fmaxf(red[tid], red[tid + h]);
        __syncthreads();
    }
    amax = red[0];
    const float sw = amax / qmax;
    for (int j = tid; j < d_in; j += 256) {
        const float v = s ? row[j] * s[j] : row[j];
        const float c = amax > 0.0f ? fminf(fmaxf(rintf(v / sw), -qmax), qmax) : 0.0f;
        float wq = sw * c;
        if (s) wq = wq / s[j];
        out[j] = row[j] - wq;
    }
}

// --------------------------------------------------------------------- channel RMS
constexpr int RMS_TOK = 256;  // tokens per partial sum

__global__ __launch_bounds__(256) void channel_sumsq_kernel(const void* __restrict__ x, int x_dtype, int T, int d_in,
                                                            double* __restrict__ part) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= d_in) return;
    const int t0 = blockIdx.y * RMS_TOK, t1 = min(T, t0 + RMS_TOK);
    double acc = 0.0;
    if (x_dtype == QE_BF16) {
        const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
        for (int t = t0; t < t1; ++t) {
            const float v = __uint_as_float((uint32_t)xb[(size_t)t * d_in + j] << 16);
            acc += (double)v * (double)v;
        }
    } else {
        const float* xf = reinterpret_cast<const float*>(x);
        for (int t = t0; t < t1; ++t) {
            const float v = xf[(size_t)t * d_in + j];
            acc += (double)v * (double)v;
        }
    }
    part[(size_t)blockIdx.y * d_in + j] = acc;
}

__global__ __launch_bounds__(256) void channel_rms_finish_kernel(const double* __restrict__ part, int nb, int T,
                                                                 int d_in, float* __restrict__ c) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= d_in) return;
    double sum = 0.0;
    for (int y = 0; y < nb; ++y) sum += part[(size_t)y * d_in + j];
    c[j] = (float)sqrt(sum / T);
}

// ------------------------------------------------------------------ thin products
constexpr int TH_A = 64;  // output rows per workgroup
constexpr int TH_B = 32;  // contraction chunk

// TRANS == false: C[a][l] += sum_b E[a][b] w[b] S[b][l]   (a < d_out, b < d_in): Z = M^T S
// TRANS == true : C[a][l] += w[a] sum_b E[b][a] S[b][l]   (a < d_in, b < d_out): Y = M S
// S [n_b][k], C [n_a][k] row-major float32, k <= KP; C is zeroed by the caller.  Each thread
// owns 4 rows x KP/16 columns; the contraction range of blockIdx.y is [y bpb, (y+1) bpb).
template <int KP, bool TRANS>
__global__ __launch_bounds__(256) void thin_kernel(const float* __restrict__ E, int d_out, int d_in,
                                                   const float* __restrict__ S, int k, const float* __restrict__ w,
                                                   int bpb, float* __restrict__ C) {
    __shared__ float Et[TH_B][TH_A + 4];  // [b][a]
    __shared__ float St[TH_B][KP];
    constexpr int LU = KP / 16;
    const int n_a = TRANS ? d_in : d_out, n_b = TRANS ? d_out : d_in;
    const int a0 = blockIdx.x * TH_A;
    const int b_beg = blockIdx.y * bpb, b_end = min(n_b, b_beg + bpb);
    const int tid = threadIdx.x, ag = tid >> 4, lg = tid & 15;
    float acc[4][LU];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int u = 0; u < LU; ++u) acc[r][u] = 0.0f;

    for (int b0 = b_beg; b0 < b_end; b0 += TH_B) {
        if constexpr (!TRANS) {  // rows a of E, 8 contiguous b per thread
            const int ar = tid >> 2, bs = (tid & 3) * 8, a = a0 + ar;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int b = b0 + bs + q;
                Et[bs + q][ar] = (a < n_a && b < b_end) ? E[(size_t)a * d_in + b] : 0.0f;
            }
        } else {  // rows b of E, 8 contiguous a per thread
            const int br = tid >> 3, as = (tid & 7) * 8, b = b0 + br;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int a = a0 + as + q;
                Et[br][as + q] = (b < b_end && a < n_a) ? E[(size_t)b * d_in + a] : 0.0f;
            }
        }
        for (int e = tid; e < TH_B * KP; e += 256) {
            const int br = e / KP, l = e % KP, b = b0 + br;
            float v = (b < b_end && l < k) ? S[(size_t)b * k + l] : 0.0f;
            if (!TRANS && w != nullptr && b < b_end) v *= w[b];
            St[br][l] = v;
        }
        __syncthreads();
#pragma unroll 4
        for (int bi = 0; bi < TH_B; ++bi) {
            float ea[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ea[r] = Et[bi][ag * 4 + r];
#pragma unroll
            for (int u = 0; u < LU; ++u) {
                const float sv = St[bi][lg + 16 * u];
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r][u] += ea[r] * sv;
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int a = a0 + ag * 4 + r;
        if (a >= n_a) continue;
        const float wa = (TRANS && w != nullptr) ? w[a] : 1.0f;
#pragma unroll
        for (int u = 0; u < LU; ++u) {
            const int l = lg + 16 * u;
            if (l < k) atomicAdd(&C[(size_t)a * k + l], acc[r][u] * wa);
        }
    }
}

__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0.0f;
}

// ------------------------------------------------------------- rank-r subtraction
// E[i][j] -= sum_l A[j][l] B[l][i]: 64 x 64 tiles of E, A and B slices in LDS, 4 x 4 per thread.
__global__ __launch_bounds__(256) void sub_lowrank_kernel(float* __restrict__ E, int d_out, int d_in,
                                                          const float* __restrict__ A, const float* __restrict__ B,
                                                          int r) {
    __shared__ float At[64][65];  // [j][l]
    __shared__ float Bt[64][65];  // [l][i]
    const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64, tid = threadIdx.x;
    for (int e = tid; e < 64 * 64; e += 256) {
        const int jj = e >> 6, l = e & 63;
        At[jj][l] = (j0 + jj < d_in && l < r) ? A[(size_t)(j0 + jj) * r + l] : 0.0f;
        const int l2 = e >> 6, ii = e & 63;
        Bt[l2][ii] = (l2 < r && i0 + ii < d_out) ? B[(size_t)l2 * d_out + i0 + ii] : 0.0f;
    }
    __syncthreads();
    const int ty = tid >> 4, tx = tid & 15;
    float acc[4][4] = {};
    for (int l = 0; l < r; ++l) {
        float bi[4], aj[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            bi[q] = Bt[l][ty * 4 + q];
            aj[q] = At[tx * 4 + q][l];
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] += aj[b] * bi[a];
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int i = i0 + ty * 4 + a;
        if (i >= d_out) continue;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int j = j0 + tx * 4 + b;
            if (j < d_in) E[(size_t)i * d_in + j] -= acc[a][b];
        }
    }
}

// C = thin product (see thin_kernel), zeroing C first
hipError_t thin(bool trans, const float* E, int d_out, int d_in, const float* S, int k, const float* w, float* C,
                hipStream_t st) {
    const int n_a = trans ? d_in : d_out, n_b = trans ? d_out : d_in;
    const size_t nc = (size_t)n_a * k;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)std::min<size_t>((nc + 255) / 256, 4096)), dim3(256), 0, st, C, nc);
    const int tiles = (n_a + TH_A - 1) / TH_A;
    const int chunks = (n_b + TH_B - 1) / TH_B;
    // about 2048 workgroups, at least 8 contraction chunks each
    const int splits = std::max(1, std::min((2048 + tiles - 1) / tiles, chunks / 8));
    const int bpb = (chunks + splits - 1) / splits * TH_B;
    const int ny = (n_b + bpb - 1) / bpb;
    const dim3 grid(tiles, ny);
#define QE_THIN(KPV)                                                                                                \
    do {                                                                                                            \
        if (trans) hipLaunchKernelGGL((thin_kernel<KPV, true>), grid, dim3(256), 0, st, E, d_out, d_in, S, k, w, bpb, C); \
        else hipLaunchKernelGGL((thin_kernel<KPV, false>), grid, dim3(256), 0, st, E, d_out, d_in, S, k, w, bpb, C); \
    } while (0)
    if (k <= 32) QE_THIN(32);
    else if (k <= 64) QE_THIN(64);
    else QE_THIN(128);
#undef QE_THIN
    return hipGetLastError();
}

// ------------------------------------------------------------------ host: thin QR
// Orthonormal basis of the columns of Y (row-major [m][n], m >= n, float32 from the device)
// by Householder reflections in double, written row-major to Q (double) and Qf (float32).
// Work is column-major; the updates of the trailing columns are split over threads.
void householder_q(const float* Y, int m, int n, double* Q, float* Qf) {
    std::vector<double> a((size_t)m * n), q((size_t)m * n, 0.0), beta(n, 0.0);
    for (int i = 0; i < m; ++i)
        for (int j = 0; j < n; ++j) a[(size_t)j * m + i] = Y[(size_t)i * n + j];
    const int n_thr = std::max(1, std::min<int>((int)std::thread::hardware_concurrency(), 8));
    auto parallel_cols = [&](int c0, int c1, auto&& fn) {  // fn(c) for c in [c0, c1)
        const long work = (long)(c1 - c0) * (m - 0);
        if (work < (1L << 18) || n_thr == 1) {
            for (int c = c0; c < c1; ++c) fn(c);
            return;
        }
        std::vector<std::thread> th;
        const int per = (c1 - c0 + n_thr - 1) / n_thr;
        for (int t = 0; t < n_thr; ++t) {
            const int b = c0 + t * per, e = std::min(c1, b + per);
            if (b >= e) break;
            th.emplace_back([&, b, e] {
                for (int c = b; c < e; ++c) fn(c);
            });
        }
        for (auto& t : th) t.join();
    };
    for (int j = 0; j < n; ++j) {
        double* v = &a[(size_t)j * m];
        double nrm = 0.0;
        for (int i = j; i < m; ++i) nrm += v[i] * v[i];
        nrm = std::sqrt(nrm);
        if (nrm == 0.0) continue;  // a zero column: no reflection
        const double alpha = v[j] >= 0.0 ? -nrm : nrm;
        v[j] -= alpha;
        double vv = 0.0;
        for (int i = j; i < m; ++i) vv += v[i] * v[i];
        beta[j] = 2.0 / vv;
        parallel_cols(j + 1, n, [&](int c) {
            double* col = &a[(size_t)c * m];
            double dot = 0.0;
            for (int i = j; i < m; ++i) dot += v[i] * col[i];
            const double f = beta[j] * dot;
            for (int i = j; i < m; ++i) col[i] -= f * v[i];
        });
    }
    // Q = H_0 ... H_{n-1} [I; 0], applied from the last reflection; columns below c < j stay zero
    for (int c = 0; c < n; ++c) q[(size_t)c * m + c] = 1.0;
    for (int j = n - 1; j >= 0; --j) {
        if (beta[j] == 0.0) continue;
        const double* v = &a[(size_t)j * m];
        parallel_cols(j, n, [&](int c) {
            double* col = &q[(size_t)c * m];
            double dot = 0.0;
            for (int i = j; i < m; ++i) dot += v[i] * col[i];
            const double f = beta[j] * dot;
            for (int i = j; i < m; ++i) col[i] -= f * v[i];
        });
    }
    for (int i = 0; i < m; ++i)
        for (int j = 0; j < n; ++j) {
            const double x = q[(size_t)j * m + i];
            if (Q) Q[(size_t)i * n + j] = x;
            Qf[(size_t)i * n + j] = (float)x;
        }
}

}  // namespace

hipError_t launch_quant_error(const float* W_f, const float* s, int d_out, int d_in, int w_bits, float* E,
                              hipStream_t st) {
    hipLaunchKernelGGL(quant_error_kernel, dim3(d_out), dim3(256), 0, st, W_f, s, d_in, w_bits == 4 ? 7.0f : 3.0f, E);
    return hipGetLastError();
}

size_t channel_rms_workspace_bytes(int T, int d_in) {
    return (size_t)((T + RMS_TOK - 1) / RMS_TOK) * d_in * sizeof(double);
}

hipError_t launch_channel_rms(const void* x, int x_dtype, int T, int d_in, float* c, void* ws, hipStream_t st) {
    const int nb = (T + RMS_TOK - 1) / RMS_TOK;
    double* part = static_cast<double*>(ws);
    hipLaunchKernelGGL(channel_sumsq_kernel, dim3((d_in + 255) / 256, nb), dim3(256), 0, st, x, x_dtype, T, d_in,
                       part);
    hipLaunchKernelGGL(channel_rms_finish_kernel, dim3((d_in + 255) / 256), dim3(256), 0, st, part, nb, T, d_in, c);
    return hipGetLastError();
}

hipError_t launch_sub_lowrank(float* E, int d_out, int d_in, const float* A, const float* B, int r, hipStream_t st) {
    hipLaunchKernelGGL(sub_lowrank_kernel, dim3((d_in + 63) / 64, (d_out + 63) / 64), dim3(256), 0, st, E, d_out,
                       d_in, A, B, r);
    return hipGetLastError();
}

// device workspace: Y / Q [d_in][k], Z / Q~ [d_out][k] (float32)
size_t lowrank_workspace_bytes(int d_out, int d_in, int k) {
    return ((size_t)2 * d_in * k + (size_t)2 * d_out * k) * sizeof(float);
}

hipError_t lowrank_fit(const float* E, int d_out, int d_in, const float* w, const float* omega, int k, int rank,
                       int power_iters, float* A, float* B, double* sigma, void* ws, hipStream_t st) {
    float* Yd = static_cast<float*>(ws);
    float* Qd = Yd + (size_t)d_in * k;
    float* Zd = Qd + (size_t)d_in * k;
    float* Qtd = Zd + (size_t)d_out * k;
    std::vector<float> hf((size_t)std::max(d_in, d_out) * k), qf((size_t)std::max(d_in, d_out) * k);
    std::vector<double> Qh((size_t)d_in * k), Zh((size_t)d_out * k);
    hipError_t e;
#define QE_TRY(expr)                          \
    do {                                      \
        if ((e = (expr)) != hipSuccess) return e; \
    } while (0)
    // orthonormal basis of a device [m][k] matrix, back on the device in `dst`
    auto orth = [&](const float* src, int m, float* dst, double* keep) -> hipError_t {
        hipError_t r;
        if ((r = hipMemcpyAsync(hf.data(), src, (size_t)m * k * sizeof(float), hipMemcpyDeviceToHost, st)) != hipSuccess)
            return r;
        if ((r = hipStreamSynchronize(st)) != hipSuccess) return r;
        householder_q(hf.data(), m, k, keep, qf.data());
        if ((r = hipMemcpyAsync(dst, qf.data(), (size_t)m * k * sizeof(float), hipMemcpyHostToDevice, st)) != hipSuccess)
            return r;
        return hipStreamSynchronize(st);  // qf is reused by the next call
    };
    QE_TRY(thin(true, E, d_out, d_in, omega, k, w, Yd, st));  // Y = M omega
    QE_TRY(orth(Yd, d_in, Qd, Qh.data()));
    for (int it = 0; it < power_iters; ++it) {
        QE_TRY(thin(false, E, d_out, d_in, Qd, k, w, Zd, st));  // M^T Q
        QE_TRY(orth(Zd, d_out, Qtd, nullptr));
        QE_TRY(thin(true, E, d_out, d_in, Qtd, k, w, Yd, st));  // M Q~
        QE_TRY(orth(Yd, d_in, Qd, Qh.data()));
    }
    QE_TRY(thin(false, E, d_out, d_in, Qd, k, w, Zd, st));  // Z = M^T Q = B^T
    QE_TRY(hipMemcpyAsync(hf.data(), Zd, (size_t)d_out * k * sizeof(float), hipMemcpyDeviceToHost, st));
    QE_TRY(hipStreamSynchronize(st));
#undef QE_TRY
    for (size_t i = 0; i < (size_t)d_out * k; ++i) Zh[i] = hf[i];

    // B B^T = Z^T Z = U~ S^2 U~^T (eigenvalues ascending from the solver)
    std::vector<double> G((size_t)k * k, 0.0), lam(k), Ut((size_t)k * k);
    for (int i = 0; i < d_out; ++i) {
        const double* z = &Zh[(size_t)i * k];
        for (int a = 0; a < k; ++a)
            for (int b = 0; b <= a; ++b) G[(size_t)a * k + b] += z[a] * z[b];
    }
    for (int a = 0; a < k; ++a)
        for (int b = a + 1; b < k; ++b) G[(size_t)a * k + b] = G[(size_t)b * k + a];
    if (symmetric_eigen(G.data(), k, lam.data(), Ut.data()) != 0) return hipErrorNotSupported;  // no convergence
    std::vector<float> wv;
    if (w) {
        wv.resize(d_in);
        if ((e = hipMemcpyAsync(wv.data(), w, (size_t)d_in * sizeof(float), hipMemcpyDeviceToHost, st)) != hipSuccess)
            return e;
        if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
    }
    std::vector<double> u(d_in), v(d_out);
    for (int l = 0; l < rank; ++l) {
        const int c = k - 1 - l;  // l-th largest
        const double s2 = std::max(lam[c], 0.0), sg = std::sqrt(s2), root = std::sqrt(sg);
        sigma[l] = sg;
        for (int j = 0; j < d_in; ++j) {
            double acc = 0.0;
            for (int a = 0; a < k; ++a) acc += Qh[(size_t)j * k + a] * Ut[(size_t)a * k + c];
            const double wj = w ? (double)wv[j] : 1.0;
            A[(size_t)j * rank + l] = wj > 0.0 ? (float)(acc / wj * root) : 0.0f;
        }
        for (int i = 0; i < d_out; ++i) {
            double acc = 0.0;
            for (int a = 0; a < k; ++a) acc += Zh[(size_t)i * k + a] * Ut[(size_t)a * k + c];
            B[(size_t)l * d_out + i] = sg > 0.0 ? (float)(acc / sg * root) : 0.0f;
        }
    }
    return hipSuccess;
}


size_t build_experts_workspace_bytes(int d_out, int d_in, int k, int r_max) {
    return align256((size_t)d_out * d_in * sizeof(float)) + align256(lowrank_workspace_bytes(d_out, d_in, k)) +
           align256((size_t)d_in * sizeof(float)) + align256((size_t)d_in * r_max * sizeof(float)) +
           align256((size_t)r_max * d_out * sizeof(float));
}

// The SE on the whole quantization error (weights c), then each RE on the residual with the
// weights of its cluster's channels only.  Host outputs; synchronizes `st`.
hipError_t build_experts(const float* W_f, const float* s, int d_out, int d_in, int w_bits, const float* c,
                         const int32_t* dep, const int32_t* labels, int n_dep, int n_r, int r_s, int r_r,
                         const float* omegas, int k, int power_iters, float* A_s, float* B_s, float* A_r, float* B_r,
                         double* sigma_s, double* sigma_r, void* ws, hipStream_t st) {
    const int r_max = std::max(r_s, r_r);
    char* p = static_cast<char*>(ws);
    float* E = reinterpret_cast<float*>(p);
    p += align256((size_t)d_out * d_in * sizeof(float));
    void* lws = p;
    p += align256(lowrank_workspace_bytes(d_out, d_in, k));
    float* wd = reinterpret_cast<float*>(p);
    p += align256((size_t)d_in * sizeof(float));
    float* Ad = reinterpret_cast<float*>(p);
    p += align256((size_t)d_in * r_max * sizeof(float));
    float* Bd = reinterpret_cast<float*>(p);
    hipError_t e;
#define QE_TRY(expr)                              \
    do {                                          \
        if ((e = (expr)) != hipSuccess) return e; \
    } while (0)
    QE_TRY(launch_quant_error(W_f, s, d_out, d_in, w_bits, E, st));
    if (r_s > 0) {
        QE_TRY(lowrank_fit(E, d_out, d_in, c, omegas, k, r_s, power_iters, A_s, B_s, sigma_s, lws, st));
        QE_TRY(hipMemcpyAsync(Ad, A_s, (size_t)d_in * r_s * sizeof(float), hipMemcpyHostToDevice, st));
        QE_TRY(hipMemcpyAsync(Bd, B_s, (size_t)r_s * d_out * sizeof(float), hipMemcpyHostToDevice, st));
        QE_TRY(launch_sub_lowrank(E, d_out, d_in, Ad, Bd, r_s, st));  // E_1 = E - (A_s B_s)^T
    }
    if (n_r > 0) {
        std::vector<float> ch(d_in), wg(d_in);
        QE_TRY(hipMemcpyAsync(ch.data(), c, (size_t)d_in * sizeof(float), hipMemcpyDeviceToHost, st));
        QE_TRY(hipStreamSynchronize(st));
        for (int g = 0; g < n_r; ++g) {
            std::fill(wg.begin(), wg.end(), 0.0f);
            for (int t = 0; t < n_dep; ++t)
                if (labels[t] == g) wg[dep[t]] = ch[dep[t]];
            QE_TRY(hipMemcpyAsync(wd, wg.data(), (size_t)d_in * sizeof(float), hipMemcpyHostToDevice, st));
            QE_TRY(hipStreamSynchronize(st));  // wg is refilled for the next cluster
            QE_TRY(lowrank_fit(E, d_out, d_in, wd, omegas + (size_t)(1 + g) * d_out * k, k, r_r, power_iters,
                               A_r + (size_t)g * d_in * r_r, B_r + (size_t)g * r_r * d_out, sigma_r + (size_t)g * r_r,
                               lws, st));
        }
    }
    QE_TRY(hipStreamSynchronize(st));
#undef QE_TRY
    return hipSuccess;
}

}  // namespace qe
