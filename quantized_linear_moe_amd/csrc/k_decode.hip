// Weight-only (A16) path of a QE linear for few tokens (decode): the packed
// weights are streamed once from HBM and multiplied with bf16 activations on
// bf16 MFMA; the dequantization and the shared / routed low-rank terms are
// applied in a split-K reduction kernel.
//
//   y[t][i] = s_w[i] * sum_j bf16(x)[t][j] * q_w[i][j] + u[t].B_s[:,i] + v[t].B_{e_t}[:,i]
//
// W3A16 is one of the pages' settings (thelatestinai.com listing, Tables 1-2 text
// and Table 8; MCISLAB DeepRead summary, "Key Results").  Codes are small
// integers, exact in bf16, so the product is exact up to float32 accumulation.
//
// Design: a workgroup owns 128 output channels (8 MFMA N blocks) and a K range;
// its 4 waves split that K range (interleaved 128-wide blocks) and reduce their
// accumulators through LDS, so one float32 partial per (K split, token,
// channel) leaves the workgroup.  Tokens (<= 16 per pass) form the MFMA M side;
// the token tile of x for the workgroup's K range is staged in LDS once.

#include "qe_internal.h"

namespace qe {

constexpr int SK_NB = 8;             // 16-channel blocks per workgroup
constexpr int SK_MAX_KBLK = 16;      // max 128-wide K blocks per workgroup
constexpr int SK_LD = SK_MAX_KBLK * 128 * 2 + 16;  // LDS row stride (bytes) of the x tile

__device__ inline uint32_t pack_bf16_pair_from_int(int lo, int hi) {
    // small integers are exact in bf16: take the upper half of the float32 bits
    const uint32_t a = __float_as_uint((float)lo), b = __float_as_uint((float)hi);
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// 8 bf16 weight values of MFMA step s (0..3) from a lane's 128-K fragment
template <int WB>
__device__ inline v8bf weight_frag(const uint32_t* f, int s) {
    v4u r;
    if (WB == 3) {
        // 32 three-bit codes, code i at bits 3i of the 96-bit value f[0..2]; step s uses codes 8s..8s+7
        const uint64_t lo = (uint64_t)f[0] | ((uint64_t)f[1] << 32);
        const uint64_t hi = (uint64_t)f[1] | ((uint64_t)f[2] << 32);
        const uint32_t field = s == 0 ? (uint32_t)lo : s == 1 ? (uint32_t)(lo >> 24) : s == 2 ? (uint32_t)(hi >> 16)
                                                                                       : (uint32_t)(f[2] >> 8);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int c0 = ((int)(field << (29 - 6 * p))) >> 29;
            const int c1 = ((int)(field << (26 - 6 * p))) >> 29;
            r[p] = pack_bf16_pair_from_int(c0, c1);
        }
    } else {
        // 4-bit tiled layout: dword s holds codes 8h..8h+7 of this step, byte b = code b | code b+4 << 4
        const uint32_t d = f[s];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int m0 = 2 * p, m1 = 2 * p + 1;
            const int sh0 = m0 < 4 ? 8 * m0 : 8 * (m0 - 4) + 4;
            const int sh1 = m1 < 4 ? 8 * m1 : 8 * (m1 - 4) + 4;
            const int c0 = ((int)(d << (28 - sh0))) >> 28;
            const int c1 = ((int)(d << (28 - sh1))) >> 28;
            r[p] = pack_bf16_pair_from_int(c0, c1);
        }
    }
    return *reinterpret_cast<v8bf*>(&r);
}

// offset (in elements, inside a 128-K block) of the 8 activations a lane feeds to MFMA step s
template <int WB>
__device__ inline int x_step_offset(int s, int lg) {
    return WB == 3 ? s * 32 + lg * 8 : (s >> 1) * 64 + lg * 16 + (s & 1) * 8;
}

template <int WB>
__global__ __launch_bounds__(256) void skinny_kernel(const void* __restrict__ x, int x_dtype, int T, int t0, int d_in,
                                                     int d_out, const uint32_t* __restrict__ w_tiled, int ksplit,
                                                     float* __restrict__ part) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t* xs = smem;                          // [16][SK_LD] x tile
    float* red = reinterpret_cast<float*>(smem);  // [4][SK_NB][64][4], reuses the x tile after the main loop
    const int NB = d_out >> 4, KB = d_in >> 7;
    const int grp = blockIdx.x, ks = blockIdx.y;
    const int kb0 = (int)((long)ks * KB / ksplit), kb1 = (int)((long)(ks + 1) * KB / ksplit);
    const int nkb = kb1 - kb0;
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int ntok = min(16, T - t0);

    // stage x[t0 .. t0+16)[kb0*128 .. kb1*128) as bf16 (zero rows beyond T)
    const int kc = nkb * 128;
    for (int i = tid; i < 16 * (kc / 8); i += 256) {
        const int r = i / (kc / 8), c8 = i % (kc / 8);
        v4u val = v4u{0, 0, 0, 0};
        if (r < ntok) {
            const size_t idx = (size_t)(t0 + r) * d_in + (size_t)kb0 * 128 + c8 * 8;
            if (x_dtype == QE_BF16) {
                val = *reinterpret_cast<const v4u*>(reinterpret_cast<const uint16_t*>(x) + idx);
            } else {
                const v4f* p = reinterpret_cast<const v4f*>(reinterpret_cast<const float*>(x) + idx);
                v4f a = p[0], b = p[1];
                auto cvt = [](float f) {
                    uint32_t u = __float_as_uint(f);
                    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
                };
                val[0] = cvt(a[0]) | (cvt(a[1]) << 16);
                val[1] = cvt(a[2]) | (cvt(a[3]) << 16);
                val[2] = cvt(b[0]) | (cvt(b[1]) << 16);
                val[3] = cvt(b[2]) | (cvt(b[3]) << 16);
            }
        }
        *reinterpret_cast<v4u*>(xs + r * SK_LD + c8 * 16) = val;
    }
    __syncthreads();

    constexpr int FW = WB == 3 ? 3 : 4;  // dwords per lane per 128-K block
    v4f acc[SK_NB];
#pragma unroll
    for (int j = 0; j < SK_NB; ++j) acc[j] = v4f{0, 0, 0, 0};

    for (int kb = kb0 + wid; kb < kb1; kb += 4) {
        uint32_t f[SK_NB][FW];
#pragma unroll
        for (int j = 0; j < SK_NB; ++j) {
            const int nb = grp * SK_NB + j;
            if (nb < NB) {
                const uint32_t* p = w_tiled + (((size_t)nb * KB + kb) * 64 + lane) * FW;
#pragma unroll
                for (int q = 0; q < FW; ++q) f[j][q] = p[q];
            } else {
#pragma unroll
                for (int q = 0; q < FW; ++q) f[j][q] = 0;
            }
        }
        const uint8_t* xrow = xs + lr * SK_LD + (kb - kb0) * 256;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const v8bf a = *reinterpret_cast<const v8bf*>(xrow + x_step_offset<WB>(s, lg) * 2);
#pragma unroll
            for (int j = 0; j < SK_NB; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, weight_frag<WB>(f[j], s), acc[j], 0, 0, 0);
        }
    }
    // reduce the 4 waves' accumulators (fixed order) through LDS
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SK_NB; ++j)
        *reinterpret_cast<v4f*>(red + ((wid * SK_NB + j) * 64 + lane) * 4) = acc[j];
    __syncthreads();
    if (wid == 0) {
        float* out = part + (size_t)ks * T * d_out;
#pragma unroll
        for (int j = 0; j < SK_NB; ++j) {
            v4f s = *reinterpret_cast<const v4f*>(red + ((0 * SK_NB + j) * 64 + lane) * 4);
#pragma unroll
            for (int w = 1; w < 4; ++w) {
                const v4f o = *reinterpret_cast<const v4f*>(red + ((w * SK_NB + j) * 64 + lane) * 4);
                s += o;
            }
            const int nb = grp * SK_NB + j;
            if (nb >= NB) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tt = lg * 4 + r;
                if (tt < ntok) out[(size_t)(t0 + tt) * d_out + nb * 16 + lr] = s[r];
            }
        }
    }
}

size_t skinny_lds_bytes() {
    static_assert(4 * SK_NB * 64 * 4 * sizeof(float) <= 16 * SK_LD, "reduction buffer must fit in the x tile");
    return 16 * SK_LD;
}

int skinny_ksplit(int d_in, int d_out) {
    const int KB = d_in / 128;
    const int groups = (d_out / 16 + SK_NB - 1) / SK_NB;
    int ks = (768 + groups - 1) / groups;
    ks = max(ks, (KB + SK_MAX_KBLK - 1) / SK_MAX_KBLK);
    ks = min(ks, KB);
    return max(ks, 1);
}

hipError_t launch_skinny(const void* x, int x_dtype, int T, int d_in, int d_out, int w_bits, const void* w_tiled,
                         int ksplit, float* part, hipStream_t st) {
    const int groups = (d_out / 16 + SK_NB - 1) / SK_NB;
    const size_t lds = skinny_lds_bytes();
    for (int t0 = 0; t0 < T; t0 += 16) {
        if (w_bits == 3) {
            hipLaunchKernelGGL(skinny_kernel<3>, dim3(groups, ksplit), dim3(256), lds, st, x, x_dtype, T, t0, d_in,
                               d_out, reinterpret_cast<const uint32_t*>(w_tiled), ksplit, part);
        } else {
            hipLaunchKernelGGL(skinny_kernel<4>, dim3(groups, ksplit), dim3(256), lds, st, x, x_dtype, T, t0, d_in,
                               d_out, reinterpret_cast<const uint32_t*>(w_tiled), ksplit, part);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t skinny_set_attributes() {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(skinny_kernel<3>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)skinny_lds_bytes());
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(skinny_kernel<4>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)skinny_lds_bytes());
}

// y[t][i] = s_w[i] * sum_ks part + u[t].Bt_s[i] + v[t].Bt_r[e_t][i]   (one thread per output)
__global__ __launch_bounds__(256) void skinny_finish_kernel(const float* __restrict__ part, int ksplit, int T,
                                                            int d_out, const float* __restrict__ w_scale,
                                                            const uint16_t* __restrict__ u,
                                                            const uint16_t* __restrict__ bt_s, int rs_pad,
                                                            const uint16_t* __restrict__ v,
                                                            const int32_t* __restrict__ expert,
                                                            const uint16_t* __restrict__ bt_r, int rr_pad,
                                                            float* __restrict__ y) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)T * d_out) return;
    const int t = (int)(idx / d_out), i = (int)(idx % d_out);
    float s = 0.0f;
    for (int k = 0; k < ksplit; ++k) s += part[((size_t)k * T + t) * d_out + i];
    float out = s * w_scale[i];
    if (u) {
        float a = 0.0f;
        for (int m = 0; m < rs_pad; ++m)
            a = __builtin_fmaf(__uint_as_float((uint32_t)u[(size_t)t * rs_pad + m] << 16),
                               __uint_as_float((uint32_t)bt_s[(size_t)i * rs_pad + m] << 16), a);
        out += a;
    }
    if (v && expert) {
        const int e = expert[t];  // produced by the router: 0 <= e < n_routed
        float a = 0.0f;
        for (int m = 0; m < rr_pad; ++m)
            a = __builtin_fmaf(__uint_as_float((uint32_t)v[(size_t)t * rr_pad + m] << 16),
                               __uint_as_float((uint32_t)bt_r[((size_t)e * d_out + i) * rr_pad + m] << 16), a);
        out += a;
    }
    y[idx] = out;
}

hipError_t launch_skinny_finish(const float* part, int ksplit, int T, int d_out, const float* w_scale,
                                const uint16_t* u, const uint16_t* bt_s, int rs_pad, const uint16_t* v,
                                const int32_t* expert, const uint16_t* bt_r, int rr_pad, float* y, hipStream_t st) {
    const size_t n = (size_t)T * d_out;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(skinny_finish_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, ksplit, T,
                       d_out, w_scale, u, bt_s, rs_pad, v, expert, bt_r, rr_pad, y);
    return hipGetLastError();
}

// Unfused routed experts, grouped by expert bucket: thread per (bucket position, channel);
// y[perm[p]][i] += v[perm[p]] . Bt_r[e][i] with e the bucket of position p.
__global__ __launch_bounds__(256) void routed_lora_kernel(const uint16_t* __restrict__ v, int rr_pad,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ perm, int n_r,
                                                          const uint16_t* __restrict__ bt_r, int T, int d_out,
                                                          float* __restrict__ y) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int p = blockIdx.y;
    if (i >= d_out || p >= T) return;
    int e = 0;
    while (e + 1 < n_r && offsets[e + 1] <= p) ++e;
    const int t = min(max(perm[p], 0), T - 1);
    float a = 0.0f;
    for (int m = 0; m < rr_pad; ++m)
        a = __builtin_fmaf(__uint_as_float((uint32_t)v[(size_t)t * rr_pad + m] << 16),
                           __uint_as_float((uint32_t)bt_r[((size_t)e * d_out + i) * rr_pad + m] << 16), a);
    y[(size_t)t * d_out + i] += a;
}

hipError_t launch_routed_lora(const uint16_t* v, int rr_pad, const int32_t* offsets, const int32_t* perm, int n_r,
                              const uint16_t* bt_r, int T, int d_out, float* y, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(routed_lora_kernel, dim3((d_out + 255) / 256, T), dim3(256), 0, st, v, rr_pad, offsets, perm,
                       n_r, bt_r, T, d_out, y);
    return hipGetLastError();
}

}  // namespace qe
