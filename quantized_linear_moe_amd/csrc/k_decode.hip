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

#include <algorithm>

#include "qe_internal.h"

namespace qe {

constexpr int SK_NB = 8;             // 16-channel blocks per workgroup
constexpr int SK_MAX_KBLK = 16;      // max 128-wide K blocks per workgroup
constexpr int SK_LD = SK_MAX_KBLK * 128 * 2 + 16;  // LDS row stride (bytes) of the x tile

// Lane fragment of one 16-channel x 128-K weight tile, by weight format:
//   WB == 3 : 3 dwords.  Codes are sign/magnitude: dword 0 holds |c| of codes 0..15 and
//             dword 1 of codes 16..31, two bits each, code 8s+p at bits 4p + 2(s&1) of
//             dword s>>1; dword 2 holds the signs, code 8s+p at bit 4p + 3 - s.  This
//             makes 8 codes of one MFMA step an fp4 (e2m1) word in three ALU ops.
//   WB == 4 : 4 dwords: the lane's 8 bytes of the two 64-K steps of the int8-GEMM tile
//             layout (see the 4-bit prepare kernel).
//   WB == 16: bf16 rows (K-contiguous); the fragment is loaded per step (no tile layout).
template <int WB>
struct Frag {
    static constexpr int kWords = WB == 3 ? 3 : WB == 4 ? 4 : 16;
};

__device__ inline uint32_t pack_bf16_pair_from_int(int lo, int hi) {
    // small integers are exact in bf16: take the upper half of the float32 bits
    const uint32_t a = __float_as_uint((float)lo), b = __float_as_uint((float)hi);
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// 8 bf16 weight values of MFMA step s (0..3) from a lane's 128-K fragment
template <int WB>
__device__ inline v8bf weight_frag(const uint32_t* f, int s) {
    v4u r;
    if constexpr (WB == 3) {
        // fp4 e2m1 nibble (sign, 0, m1, m0) with magnitude m in {0,1,2,3} encodes m/2;
        // scaling by 2 in the conversion gives the code exactly in bf16
        const uint32_t mag = (s & 1) ? (f[s >> 1] >> 2) : f[s >> 1];
        const uint32_t fp4 = (mag & 0x33333333u) | ((f[2] << s) & 0x88888888u);
        const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(fp4, 2.0f, 0);
        const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(fp4, 2.0f, 1);
        const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(fp4, 2.0f, 2);
        const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(fp4, 2.0f, 3);
        r[0] = *reinterpret_cast<const uint32_t*>(&p0);
        r[1] = *reinterpret_cast<const uint32_t*>(&p1);
        r[2] = *reinterpret_cast<const uint32_t*>(&p2);
        r[3] = *reinterpret_cast<const uint32_t*>(&p3);
    } else if constexpr (WB == 4) {
        // 4-bit tiled layout: dword s holds this step's 8 codes, byte b = code b | code b+4 << 4
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
    } else {
        r = v4u{f[4 * s], f[4 * s + 1], f[4 * s + 2], f[4 * s + 3]};
    }
    return *reinterpret_cast<v8bf*>(&r);
}

// offset (in elements, inside a 128-K block) of the 8 activations a lane feeds to MFMA step s
template <int WB>
__device__ inline int x_step_offset(int s, int lg) {
    return WB == 4 ? (s >> 1) * 64 + lg * 16 + (s & 1) * 8 : s * 32 + lg * 8;
}

// Load one lane's fragment of K block kb for channel block nb (zeros beyond the valid blocks).
template <int WB>
__device__ inline void load_frag(const uint32_t* __restrict__ w, int nb, int NB, int kb, int KB, int lane, int d_in,
                                 uint32_t (&f)[Frag<WB>::kWords]) {
    constexpr int FW = Frag<WB>::kWords;
    if (nb >= NB) {
#pragma unroll
        for (int q = 0; q < FW; ++q) f[q] = 0;
        return;
    }
    if constexpr (WB == 3) {
        const uint32_t* p = w + (((size_t)nb * KB + kb) * 64 + lane) * 3;
        f[0] = p[0];
        f[1] = p[1];
        f[2] = p[2];
    } else if constexpr (WB == 4) {
        // two 64-K steps of the 4-bit tile layout: 8 bytes per lane each
        const v2u q0 = *reinterpret_cast<const v2u*>(w + (((size_t)nb * 2 * KB + 2 * kb) * 64 + lane) * 2);
        const v2u q1 = *reinterpret_cast<const v2u*>(w + (((size_t)nb * 2 * KB + 2 * kb + 1) * 64 + lane) * 2);
        f[0] = q0[0]; f[1] = q0[1]; f[2] = q1[0]; f[3] = q1[1];
    } else {
        // bf16 rows of d_in elements: channel nb*16 + (lane & 15), K = kb*128 + s*32 + (lane >> 4)*8
        const uint16_t* row = reinterpret_cast<const uint16_t*>(w) + (size_t)(nb * 16 + (lane & 15)) * d_in +
                              (size_t)kb * 128 + (lane >> 4) * 8;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const v4u q = *reinterpret_cast<const v4u*>(row + s * 32);
            f[4 * s] = q[0]; f[4 * s + 1] = q[1]; f[4 * s + 2] = q[2]; f[4 * s + 3] = q[3];
        }
    }
}

// part[ks][t][c] = sum over this workgroup's K range of bf16(x)[t][k] * W[c][k], for the
// token tile t0..t0+15 and channels c of its 8 channel blocks (out_ld = row stride of part).
template <int WB>
__global__ __launch_bounds__(256) void skinny_kernel(const void* __restrict__ x, int x_dtype, int T, int t0, int d_in,
                                                     int n_cols, const uint32_t* __restrict__ w_tiled, int ksplit,
                                                     float* __restrict__ part, int out_ld) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t* xs = smem;                          // [ntok][SK_LD] x tile
    float* red = reinterpret_cast<float*>(smem);  // [4][SK_NB][64][4], reuses the LDS after the main loop
    const int NB = n_cols >> 4, KB = d_in >> 7;
    const int grp = blockIdx.x, ks = blockIdx.y;
    const int kb0 = (int)((long)ks * KB / ksplit), kb1 = (int)((long)(ks + 1) * KB / ksplit);
    const int nkb = kb1 - kb0;
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int ntok = min(16, T - t0);
    constexpr int FW = Frag<WB>::kWords;

    // weight fragments of this wave's first K block are requested before the x tile is staged
    uint32_t f[SK_NB][FW], fn[SK_NB][FW];
    int kb = kb0 + wid;
    if (kb < kb1) {
#pragma unroll
        for (int j = 0; j < SK_NB; ++j) load_frag<WB>(w_tiled, grp * SK_NB + j, NB, kb, KB, lane, d_in, f[j]);
    }

    // stage x[t0 .. t0+ntok)[kb0*128 .. kb1*128) as bf16, eight independent 16-byte loads
    // per thread in flight per batch
    const int kc8 = nkb * 16;  // 16-byte chunks per row
    const int total = ntok * kc8;
    for (int base = 0; base < total; base += 256 * 8) {
        v4u val[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int i = base + q * 256 + tid;
            val[q] = v4u{0, 0, 0, 0};
            if (i < total) {
                const int r = i / kc8, c8 = i % kc8;
                const size_t idx = (size_t)(t0 + r) * d_in + (size_t)kb0 * 128 + c8 * 8;
                if (x_dtype == QE_BF16) {
                    val[q] = *reinterpret_cast<const v4u*>(reinterpret_cast<const uint16_t*>(x) + idx);
                } else {
                    const v4f* p = reinterpret_cast<const v4f*>(reinterpret_cast<const float*>(x) + idx);
                    const v4f a = p[0], b = p[1];
                    auto cvt = [](float fv) {
                        uint32_t u = __float_as_uint(fv);
                        return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
                    };
                    val[q][0] = cvt(a[0]) | (cvt(a[1]) << 16);
                    val[q][1] = cvt(a[2]) | (cvt(a[3]) << 16);
                    val[q][2] = cvt(b[0]) | (cvt(b[1]) << 16);
                    val[q][3] = cvt(b[2]) | (cvt(b[3]) << 16);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int i = base + q * 256 + tid;
            if (i < total) *reinterpret_cast<v4u*>(xs + (i / kc8) * SK_LD + (i % kc8) * 16) = val[q];
        }
    }
    __syncthreads();

    v4f acc[SK_NB];
#pragma unroll
    for (int j = 0; j < SK_NB; ++j) acc[j] = v4f{0, 0, 0, 0};

    for (; kb < kb1; kb += 4) {
        // next K block of this wave, one block ahead (the bf16 rows are 4x larger and are
        // not double-buffered, to keep two waves per SIMD)
        const bool more = WB != 16 && kb + 4 < kb1;
        if (more) {
#pragma unroll
            for (int j = 0; j < SK_NB; ++j) load_frag<WB>(w_tiled, grp * SK_NB + j, NB, kb + 4, KB, lane, d_in, fn[j]);
        }
        const uint8_t* xrow = xs + lr * SK_LD + (kb - kb0) * 256;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const v8bf a = lr < ntok ? *reinterpret_cast<const v8bf*>(xrow + x_step_offset<WB>(s, lg) * 2) : v8bf{};
#pragma unroll
            for (int j = 0; j < SK_NB; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, weight_frag<WB>(f[j], s), acc[j], 0, 0, 0);
        }
        if (more) {
#pragma unroll
            for (int j = 0; j < SK_NB; ++j)
#pragma unroll
                for (int q = 0; q < FW; ++q) f[j][q] = fn[j][q];
        } else if (WB == 16 && kb + 4 < kb1) {
#pragma unroll
            for (int j = 0; j < SK_NB; ++j) load_frag<WB>(w_tiled, grp * SK_NB + j, NB, kb + 4, KB, lane, d_in, f[j]);
        }
    }
    // reduce the 4 waves' accumulators (fixed order) through LDS
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SK_NB; ++j)
        *reinterpret_cast<v4f*>(red + ((wid * SK_NB + j) * 64 + lane) * 4) = acc[j];
    __syncthreads();
    if (wid == 0) {
        float* out = part + (size_t)ks * T * out_ld;
#pragma unroll
        for (int j = 0; j < SK_NB; ++j) {
            v4f sum = *reinterpret_cast<const v4f*>(red + ((0 * SK_NB + j) * 64 + lane) * 4);
#pragma unroll
            for (int w = 1; w < 4; ++w) {
                const v4f o = *reinterpret_cast<const v4f*>(red + ((w * SK_NB + j) * 64 + lane) * 4);
                sum += o;
            }
            const int nb = grp * SK_NB + j;
            if (nb >= NB) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tt = lg * 4 + r;
                if (tt < ntok) out[(size_t)(t0 + tt) * out_ld + nb * 16 + lr] = sum[r];
            }
        }
    }
}

constexpr size_t SK_RED_BYTES = 4 * SK_NB * 64 * 4 * sizeof(float);
size_t skinny_lds_bytes(int ntok) { return std::max((size_t)ntok * SK_LD, SK_RED_BYTES); }
size_t skinny_lds_bytes() { return skinny_lds_bytes(16); }

int skinny_ksplit(int d_in, int d_out) {
    const int KB = d_in / 128;
    const int groups = (d_out / 16 + SK_NB - 1) / SK_NB;
    if (groups <= 0 || KB <= 0) return 1;
    int ks = (1024 + groups - 1) / groups;
    ks = max(ks, (KB + SK_MAX_KBLK - 1) / SK_MAX_KBLK);
    ks = min(ks, KB);
    return max(ks, 1);
}

// K splits of the small-T x-projection: few partials per output, so its reduction stays short
int skinny_ksplit_proj(int d_in) { return std::max(1, std::min(d_in / 128, 128)); }

// w_bits 3 / 4: packed tiles; w_bits 16: bf16 rows (the x-projection matrix), n_cols columns
hipError_t launch_skinny(const void* x, int x_dtype, int T, int d_in, int n_cols, int w_bits, const void* w_tiled,
                         int ksplit, float* part, int out_ld, hipStream_t st) {
    const int groups = (n_cols / 16 + SK_NB - 1) / SK_NB;
    const uint32_t* w = reinterpret_cast<const uint32_t*>(w_tiled);
    for (int t0 = 0; t0 < T; t0 += 16) {
        const size_t lds = skinny_lds_bytes(std::min(16, T - t0));
        if (w_bits == 3) {
            hipLaunchKernelGGL(skinny_kernel<3>, dim3(groups, ksplit), dim3(256), lds, st, x, x_dtype, T, t0, d_in,
                               n_cols, w, ksplit, part, out_ld);
        } else if (w_bits == 4) {
            hipLaunchKernelGGL(skinny_kernel<4>, dim3(groups, ksplit), dim3(256), lds, st, x, x_dtype, T, t0, d_in,
                               n_cols, w, ksplit, part, out_ld);
        } else {
            hipLaunchKernelGGL(skinny_kernel<16>, dim3(groups, ksplit), dim3(256), lds, st, x, x_dtype, T, t0, d_in,
                               n_cols, w, ksplit, part, out_ld);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t skinny_set_attributes() {
    const int lds = (int)skinny_lds_bytes();
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(skinny_kernel<3>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(skinny_kernel<4>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(skinny_kernel<16>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    return e;
}

// One thread per (token t, channel i):
//   y[t][i] = s_w[i] * sum_ks part[ks][t][i] + u[t].Bt_s[i] + v[t].Bt_r[e_t][i]
// with the adapter rows read as 16-byte vectors (rows are padded to 32 elements).
__device__ inline float dot_bf16_rows(const uint16_t* __restrict__ a, const uint16_t* __restrict__ b, int n) {
    float acc = 0.0f;
    for (int m = 0; m < n; m += 8) {
        const v4u bv = *reinterpret_cast<const v4u*>(b + m);
        const v4u av = *reinterpret_cast<const v4u*>(a + m);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc = __builtin_fmaf(__uint_as_float(av[q] << 16), __uint_as_float(bv[q] << 16), acc);
            acc = __builtin_fmaf(__uint_as_float(av[q] & 0xFFFF0000u), __uint_as_float(bv[q] & 0xFFFF0000u), acc);
        }
    }
    return acc;
}

__global__ __launch_bounds__(256) void skinny_finish_kernel(const float* __restrict__ part, int ksplit, int T,
                                                            int d_out, const float* __restrict__ w_scale,
                                                            const uint16_t* __restrict__ u,
                                                            const uint16_t* __restrict__ bt_s, int rs_pad,
                                                            const uint16_t* __restrict__ v,
                                                            const int32_t* __restrict__ expert,
                                                            const uint16_t* __restrict__ bt_r, int rr_pad,
                                                            float* __restrict__ y) {
    const int i = blockIdx.x * 256 + threadIdx.x, t = blockIdx.y;
    if (i >= d_out) return;
    const float* p = part + (size_t)t * d_out + i;
    const size_t stride = (size_t)T * d_out;
    float s = 0.0f;
    int k = 0;
    for (; k + 4 <= ksplit; k += 4) {  // independent loads, summed in order
        const float a0 = p[(size_t)k * stride], a1 = p[(size_t)(k + 1) * stride];
        const float a2 = p[(size_t)(k + 2) * stride], a3 = p[(size_t)(k + 3) * stride];
        s += a0;
        s += a1;
        s += a2;
        s += a3;
    }
    for (; k < ksplit; ++k) s += p[(size_t)k * stride];
    float out = s * w_scale[i];
    if (u) out += dot_bf16_rows(u + (size_t)t * rs_pad, bt_s + (size_t)i * rs_pad, rs_pad);
    if (v && expert) out += dot_bf16_rows(v + (size_t)t * rr_pad, bt_r + ((size_t)expert[t] * d_out + i) * rr_pad, rr_pad);
    y[(size_t)t * d_out + i] = out;
}

hipError_t launch_skinny_finish(const float* part, int ksplit, int T, int d_out, const float* w_scale,
                                const uint16_t* u, const uint16_t* bt_s, int rs_pad, const uint16_t* v,
                                const int32_t* expert, const uint16_t* bt_r, int rr_pad, float* y, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(skinny_finish_kernel, dim3((d_out + 255) / 256, T), dim3(256), 0, st, part, ksplit, T, d_out,
                       w_scale, u, bt_s, rs_pad, v, expert, bt_r, rr_pad, y);
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
