// Internal declarations shared by the libqe translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/qe.h"

namespace qe {

// ------------------------------------------------------------------ vector types
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxRouted = 16;
constexpr int kMaxRank = 64;
constexpr int kRankPad = 32;  // adapter ranks are padded to a multiple of one bf16 MFMA K step

__host__ __device__ inline int rank_pad(int r) { return r <= 0 ? 0 : (r + kRankPad - 1) / kRankPad * kRankPad; }

// float32 -> bf16 bits, round to nearest even (inputs finite)
__device__ inline uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// One output element of y: float32, or bf16 (round to nearest even of the same float32 value)
// when the linear writes bf16 outputs (y then points at uint16_t elements).
__device__ inline void store_y(float* y, size_t idx, float v, bool y_bf16) {
    if (y_bf16) reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)f32_to_bf16_bits(v);
    else y[idx] = v;
}
__host__ __device__ inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// 16 four-bit weight codes of one int8-MFMA fragment (8 bytes of the tiled layout, byte b holding
// code b in the low nibble and code b+4 in the high one) as int8 values 16*code: each nibble moves
// into the high half of its byte, so no sign extension is needed and an int32 accumulator holds
// 16 * sum exactly (recovered by an arithmetic shift)
__device__ inline v4i unpack_w4x16(uint32_t p0, uint32_t p1) {
    v4i r;
    r[0] = (int)((p0 << 4) & 0xF0F0F0F0u);
    r[1] = (int)(p0 & 0xF0F0F0F0u);
    r[2] = (int)((p1 << 4) & 0xF0F0F0F0u);
    r[3] = (int)(p1 & 0xF0F0F0F0u);
    return r;
}

// ---------------------------------------------------------- prepared-buffer map
// All offsets are in bytes from the start of the prepared buffer.
struct PrepLayout {
    size_t w_tiled, w_tiled_bytes;  // main weights in the kernel layout
    size_t w_scale;                 // float [d_out]
    size_t smooth, inv_smooth;      // float [d_in] each (0 bytes when a_bits == 16)
    size_t mt;                      // bf16 [n_cols_pad][d_in]: A_s^T, R^T (16-row padded), A_1^T..A_N^T
    size_t bt_s;                    // bf16 [d_out][rs_pad]  (B_s transposed, zero padded)
    size_t bt_r;                    // bf16 [N_r][d_out][rr_pad]
    size_t total;
    int rs_pad, rr_pad;
    int col_se, col_re, col_router;  // first row of each block inside mt
    int n_lead;                      // rows of the leading block (shared expert + router)
    int n_cols, n_cols_pad;
    bool has_smooth;
};

// ---------------------------------------------------------------- workspace map
struct WsLayout {
    size_t codes;       // int8 [T][d_in]
    size_t s_x;         // float [T]
    size_t part;        // float [ksplit][T][n_cols_pad]  (x-projection partials)
    size_t scores;      // float [T][N_r]
    size_t expert;      // int32 [T]
    size_t counts;      // int32 [32]
    size_t offsets;     // int32 [32]
    size_t perm;        // int32 [T]
    size_t u;           // bf16 [T][rs_pad]
    size_t v;           // bf16 [T][rr_pad]
    size_t skinny;      // float [ksplit][T][d_out]   (decode split-K partials)
    size_t amax;        // float [rp_ksplit][T]       (route pass: partial max |x/s|)
    size_t total;
    int xproj_ksplit;
    int skinny_ksplit;
    size_t vpart;       // float [eq_ksplit][T][rr_pad] (expert-quant split-K partials)
    int rp_ksplit, eq_ksplit;  // 0 unless the two-pass prefill prologue is used
    int gemm_ksplit;           // K splits of the A6/A8 main product (partials in `skinny`)
};

PrepLayout prep_layout(const qe_linear* lin);
bool two_pass_sized(const qe_linear* lin, int T);
WsLayout ws_layout(const qe_linear* lin, int T);

// ----------------------------------------------------------- launch wrappers
// Each returns hipSuccess or the launch error.  All arguments are validated by the
// caller (qe_api.hip) before these are called.
hipError_t launch_quant_act(const void* x, int x_dtype, const float* smooth, const float* inv_smooth,
                            int T, int d_in, int a_bits, int8_t* codes, float* s_x, hipStream_t st);

hipError_t launch_xproj(const void* x, int x_dtype, int T, int d_in, const uint16_t* mt, int col0, int ncols,
                        int ncols_pad, int ksplit, float* part, hipStream_t st);

// Reduces x-projection partials; routes (if router_col >= 0) or takes `expert_in`;
// writes scores/expert and the bf16 adapter inputs u (shared) and v (selected routed).
hipError_t launch_xproj_finish(const float* part, int ksplit, int T, int ncols_pad, int col0, int se_col,
                               int r_s, int rs_pad, int re_col, int n_r, int r_r, int rr_pad, int router_col,
                               const int32_t* expert_in, float* scores, int32_t* expert_out, uint16_t* u,
                               uint16_t* v, hipStream_t st, int32_t* expert2_out = nullptr);

// two-pass prefill prologue
hipError_t launch_route_pass(const uint16_t* x, int T, int d_in, const uint16_t* mt, int ncols, const float* smooth,
                             const float* inv_smooth, int ksplit, float* part, float* amax_part, hipStream_t st);
int route_pass_ksplit(int T, int d_in);
// the route pass of up to RG_MAX linears that read the same x (one read of x): per linear its
// projection rows (Mt's leading ncols rows, ncols 16..48), smoothing factors and the partial
// buffers the single-linear pass would write
constexpr int RG_MAX = 3;
struct RouteGroup {
    const uint16_t* mt[RG_MAX];
    const float* smooth[RG_MAX];
    const float* inv_smooth[RG_MAX];
    float* part[RG_MAX];
    float* amax[RG_MAX];
    int ncols[RG_MAX];
};
hipError_t launch_route_pass_group(const uint16_t* x, int T, int d_in, const RouteGroup& G, int n_lin, int ksplit,
                                   hipStream_t st);
// the rest of the two-pass prologue for the linears of a group, each step one launch for all
// of them (route finishes; expert-sorted passes and v finishes); the same arithmetic as the
// per-linear launches
struct FinishLinear {
    const float* part;
    const float* amax;
    int ncols, r_s, rs_pad, router_col, n_r, qmax;
    int32_t* expert;
    uint16_t* u;
    float* s_x;
};
struct FinishGroup {
    FinishLinear lin[RG_MAX];
};
hipError_t launch_route_finish_group(const FinishGroup& G, int n_lin, int ksplit, int T, hipStream_t st);
// Few-token prologue in one launch (one workgroup per token, one more for u): codes, s_x, u,
// routes and v, all in token order; row_prologue_ok says which shapes it takes
bool row_prologue_ok(int T, int d_in, int rs_pad, int n_r, int rr_pad);
hipError_t launch_row_prologue(const uint16_t* x, int T, int d_in, const float* smooth, const float* inv_smooth,
                               int a_bits, const uint16_t* mt, int r_s, int rs_pad, int col_router, int n_r, int col_re,
                               int r_r, int rr_pad, int8_t* codes, float* s_x, uint16_t* u, int32_t* expert,
                               uint16_t* v, hipStream_t st);
struct EqLinear {
    const float* smooth;
    const float* inv_smooth;
    const float* s_x;
    int qmax;
    const int32_t* expert;
    int n_r;
    const uint16_t* mt_re;
    int r_r;
    int32_t* perm;
    float* vpart;
    int8_t* codes;
    uint16_t* v;
};
struct EqGroup {
    EqLinear lin[RG_MAX];
};
// every linear routed, with the same padded rank rr_pad (32 or 64)
hipError_t launch_expert_quant_group(const uint16_t* x, int T, int d_in, const EqGroup& G, int n_lin, int rr_pad,
                                     int ksq, bool keep_order, hipStream_t st);
hipError_t launch_route_finish(const float* part, const float* amax_part, int ksplit, int T, int ncols, int r_s,
                               int rs_pad, int router_col, int n_r, int a_bits, int32_t* expert, uint16_t* u,
                               float* s_x, hipStream_t st, int32_t* expert2 = nullptr);
// Expert-sorted codes + selected-expert v; buckets the routes itself and writes perm
// (needed when ksq > 1: the split-K finish scatters v through it)
hipError_t launch_expert_quant(const uint16_t* x, int T, int d_in, const float* smooth, const float* inv_smooth,
                               const float* s_x, int a_bits, const int32_t* expert, int n_r, const uint16_t* mt_re,
                               int rr_pad, int r_r, int ksq, int32_t* perm, float* vpart, int8_t* codes, uint16_t* v,
                               bool keep_order, hipStream_t st);
int expert_quant_ksplit(int T, int d_in);

hipError_t launch_second_expert(const float* scores, const int32_t* expert1, int T, int n_r, int32_t* expert2,
                                hipStream_t st);
hipError_t launch_bucket(const int32_t* expert, int T, int n_r, int32_t* counts, int32_t* offsets,
                         int32_t* perm, hipStream_t st);

// ksplit > 1 (with part: int32 [ksplit][T][d_out]) splits the K steps over workgroups and
// adds the partial sums in a finish kernel; only for grids of 64-token tiles (gemm_ksplit)
hipError_t launch_gemm_w4(const int8_t* codes, const float* s_x, const uint8_t* w_tiled, const float* w_scale,
                          int T, int d_in, int d_out, const uint16_t* u, const uint16_t* bt_s, int rs_pad,
                          const uint16_t* v, const int32_t* expert, const uint16_t* bt_r, int rr_pad, int n_r,
                          const int32_t* perm, float* y, int32_t* acc_debug, int ksplit, int32_t* part,
                          bool y_bf16, hipStream_t st);
int gemm_ksplit(int T, int d_in, int d_out);
// top-2 routing: both routed corrections in the main product's epilogue (128-token tiles, fast
// epilogue, no K split); gemm_w4_top2_ok says whether a launch of these sizes takes it
bool gemm_w4_top2_ok(int T, int d_out, int rs_pad, int rr_pad, int ksplit, bool y_bf16);
hipError_t launch_gemm_w4_top2(const int8_t* codes, const float* s_x, const uint8_t* w_tiled, const float* w_scale,
                               int T, int d_in, int d_out, const uint16_t* u, const uint16_t* bt_s, int rs_pad,
                               const uint16_t* v, const int32_t* expert, const uint16_t* v2, const int32_t* expert2,
                               const uint16_t* bt_r, int rr_pad, int n_r, const int32_t* perm, float* y,
                               hipStream_t st);
// several linears' main products (fast epilogue, float32 y, no K split) in one launch
constexpr int GG_MAX = 3;
struct GemmLinear {
    const int8_t* codes;
    const float* s_x;
    const uint8_t* w_tiled;
    const float* w_scale;
    const uint16_t* u;
    const uint16_t* bt_s;
    const uint16_t* v;
    const int32_t* expert;
    const uint16_t* bt_r;
    const int32_t* perm;
    float* y;
    int d_in, d_out, rs_pad, rr_pad, n_r;
};
struct GemmGroup {
    GemmLinear lin[GG_MAX];
    int begin[GG_MAX];
    int n, T;
};
hipError_t launch_gemm_w4_group(const GemmGroup& G, hipStream_t st);
hipError_t launch_gemm_split_finish(const int32_t* part, int ksplit, int T, int d_out, const float* s_x,
                                    const float* w_scale, const uint16_t* u, const uint16_t* bt_s, int rs_pad,
                                    const uint16_t* v, const int32_t* expert, int n_r, const uint16_t* bt_r,
                                    int rr_pad, float* y, bool y_bf16, hipStream_t st);

// weight streaming for few tokens: w_bits 3 / 4 read packed tiles, w_bits 16 reads bf16 rows
// (the x-projection matrix); part[ks][t][c] with row stride out_ld
hipError_t launch_skinny(const void* x, int x_dtype, int T, int d_in, int n_cols, int w_bits, const void* w_tiled,
                         int ksplit, float* part, int out_ld, hipStream_t st);
int skinny_ksplit(int d_in, int d_out);
int skinny_ksplit_proj(int d_in);
hipError_t launch_probe_mfma_i8(int32_t* out, int blocks, int iters, int operands, hipStream_t st);
double probe_mfma_i8_ops(int blocks, int iters);
hipError_t launch_probe_mfma_bf16(float* out, int blocks, int iters, int operands, hipStream_t st);
double probe_mfma_bf16_flops(int blocks, int iters);
hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t st);
hipError_t launch_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st);
size_t probe_read_sink_words();

// fused weight-only decode (T <= 16): one GEMV launch for the projection and the packed
// weights, one finish launch
struct DecodePlan {
    int ks_m, ks_p;      // K splits of the main weights and of the projection
    int n_mwg, n_pwg;    // workgroups of each stream
    int ld_m, ld_p;      // LDS row strides of their x tiles
    size_t lds;          // dynamic LDS bytes
};
DecodePlan decode_plan(int d_in, int d_out, int w_bits, int ncp, int T);
hipError_t launch_decode_gemv(const void* x, int x_dtype, const int8_t* codes, int T, int d_in, int d_out, int w_bits,
                              const void* w_tiled, const DecodePlan& P, float* part_m, const uint16_t* mt, int ncp,
                              float* part_p, hipStream_t st);
hipError_t launch_decode_finish(const float* part_m, const float* s_x, int ks_m, int T, int d_out,
                                const float* w_scale, const float* part_p, int ks_p, int ncp, int col_se, int r_s,
                                int rs_pad, int col_re, int n_r, int r_r, int rr_pad, int col_router,
                                const uint16_t* bt_s, const uint16_t* bt_r, int32_t* expert_out, float* y,
                                bool y_bf16, hipStream_t st);

hipError_t launch_skinny_finish(const float* part, int ksplit, int T, int d_out, const float* w_scale,
                                const uint16_t* u, const uint16_t* bt_s, int rs_pad, const uint16_t* v,
                                const int32_t* expert, const uint16_t* bt_r, int rr_pad, float* y, bool y_bf16,
                                hipStream_t st);

hipError_t launch_routed_lora(const uint16_t* v, int rr_pad, const int32_t* offsets, const int32_t* perm, int n_r,
                              const uint16_t* bt_r, int T, int d_out, float* y, hipStream_t st);

hipError_t launch_colmean(const void* W, int dtype, int d_out, int d_in, float* w, hipStream_t st);

hipError_t launch_topk(const void* x, int x_dtype, const float* w, int T, int d_in, int k, int32_t* topk,
                       uint32_t* hist, hipStream_t st);

// prepare kernels
hipError_t launch_prep_w4(const uint8_t* packed, int d_out, int d_in, uint8_t* tiled, hipStream_t st);
hipError_t launch_prep_w3(const uint32_t* packed, int d_out, int d_in, uint32_t* tiled, hipStream_t st);
hipError_t launch_prep_transpose(const uint16_t* src, int rows, int cols, uint16_t* dst, int dst_ld, int dst_rows,
                                 hipStream_t st);  // dst[c][r] = src[r][c], zero fill up to dst_rows x dst_ld
hipError_t launch_prep_smooth(const float* s, int d_in, float* s_out, float* inv_out, hipStream_t st);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);

}  // namespace qe
