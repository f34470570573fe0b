// Weight fragments of the packed layouts for bf16 (and int8) MFMAs: shared by the
// weight-streaming kernels (few tokens) and the A16 GEMM (many tokens).
#pragma once

#include "qe_internal.h"

namespace qe {

// Lane fragment of one 16-channel x 128-K weight tile, by weight format:
//   WB == 3 : 3 dwords.  Codes are sign/magnitude: dword 0 holds |c| of codes 0..15 and
//             dword 1 of codes 16..31, two bits each, code 8s+p at bits 4p + 2(s&1) of
//             dword s>>1; dword 2 holds the signs, code 8s+p at bit 4p + 3 - s.  This
//             makes 8 codes of one MFMA step an fp4 (e2m1) word in three ALU ops.
//   WB == 4 : 4 dwords: the lane's 8 bytes of the two 64-K steps of the int8-GEMM tile
//             layout (see the 4-bit prepare kernel).
//   WB == 16: bf16 rows (K-contiguous); the fragment is loaded per step (no tile layout).
//   WB == 8 : the 4-bit layout of WB == 4, multiplied with int8 activation codes.
template <int WB>
struct Frag {
    static constexpr int kWords = WB == 3 ? 3 : (WB == 4 || WB == 8) ? 4 : 16;
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
    } else if constexpr (WB == 4 || WB == 8) {
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

}  // namespace qe
