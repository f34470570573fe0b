// Host side of libqe: argument validation, buffer layouts, launch sequencing,
// weight quantization/packing (host) and the Table 7 cost model.
// See include/qe.h for the contract of every entry point.

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <thread>
#include <vector>

#include "qe_calib.h"
#include "qe_lowrank.h"
#include "qe_internal.h"

namespace qe {
hipError_t skinny_set_attributes();
// token counts for which the expert-sorted quantization pass may keep token order
bool expert_quant_few(int T);
// weight-only (A16) main product for more than 16 tokens with its epilogue (part: float
// [ksplit][T][d_out] scratch)
int gemm_a16_ksplit(int T, int d_in, int d_out, int w_bits);
hipError_t launch_gemm_a16(const void* x, int x_dtype, int T, int d_in, int d_out, int w_bits, const void* w_tiled,
                           int ksplit, float* part, const float* w_scale, const uint16_t* u, const uint16_t* bt_s,
                           int rs_pad, const uint16_t* v, const int32_t* expert, const uint16_t* bt_r, int rr_pad,
                           int n_r, float* y, bool y_bf16, hipStream_t st);
}  // namespace qe

using namespace qe;

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    return QE_ERR_HIP;
}

#define QE_TRY_HIP(expr)                            \
    do {                                            \
        hipError_t _e = (expr);                     \
        if (_e != hipSuccess) return hip_fail(_e);  \
    } while (0)

#define QE_CHECK(cond, code) \
    do {                     \
        if (!(cond)) return (code); \
    } while (0)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int validate_linear(const qe_linear* lin) {
    QE_CHECK(lin != nullptr, QE_ERR_INVALID_ARG);
    QE_CHECK(lin->d_in > 0 && lin->d_out > 0, QE_ERR_INVALID_ARG);
    QE_CHECK(lin->w_bits == 3 || lin->w_bits == 4, QE_ERR_INVALID_ARG);
    QE_CHECK(lin->a_bits == 6 || lin->a_bits == 8 || lin->a_bits == 16, QE_ERR_INVALID_ARG);
    QE_CHECK(!(lin->w_bits == 3 && lin->a_bits != 16), QE_ERR_UNSUPPORTED);
    QE_CHECK(lin->r_shared >= 0 && lin->r_shared <= kMaxRank, QE_ERR_INVALID_ARG);
    QE_CHECK(lin->n_routed >= 0 && lin->n_routed <= kMaxRouted, QE_ERR_INVALID_ARG);
    if (lin->n_routed > 0) {
        QE_CHECK(lin->r_routed >= 1 && lin->r_routed <= kMaxRank, QE_ERR_INVALID_ARG);
    } else {
        QE_CHECK(lin->r_routed == 0, QE_ERR_INVALID_ARG);
    }
    QE_CHECK(lin->y_dtype == QE_F32 || lin->y_dtype == QE_BF16, QE_ERR_INVALID_ARG);
    QE_CHECK(lin->d_out % 16 == 0, QE_ERR_UNSUPPORTED);
    QE_CHECK(lin->d_in % 128 == 0, QE_ERR_UNSUPPORTED);
    // 16 * |acc| must stay below 2^31 on the int8 path: 16 * 127 * 7 * d_in
    QE_CHECK(lin->a_bits == 16 || (int64_t)lin->d_in * 16 * 127 * 7 < (int64_t)INT32_MAX, QE_ERR_UNSUPPORTED);
    QE_CHECK(lin->a_bits == 16 || lin->d_in <= 32768, QE_ERR_UNSUPPORTED);  // one token row per workgroup
    return QE_OK;
}

int validate_forward_common(const qe_linear* lin, int32_t T, int32_t x_dtype, const void* x, void* ws,
                            size_t ws_bytes) {
    int st = validate_linear(lin);
    if (st) return st;
    QE_CHECK(T >= 0, QE_ERR_INVALID_ARG);
    QE_CHECK(x_dtype == QE_F32 || x_dtype == QE_BF16, QE_ERR_INVALID_ARG);
    QE_CHECK(lin->prep != nullptr, QE_ERR_INVALID_ARG);
    QE_CHECK(aligned16(lin->prep), QE_ERR_ALIGNMENT);
    if (x) QE_CHECK(aligned16(x), QE_ERR_ALIGNMENT);
    if (T > 0) QE_CHECK(ws_bytes >= qe_workspace_bytes(lin, T), QE_ERR_WORKSPACE);
    if (T > 0) QE_CHECK(ws != nullptr, QE_ERR_WORKSPACE);
    if (ws) QE_CHECK(aligned16(ws), QE_ERR_ALIGNMENT);
    return QE_OK;
}

inline hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

template <class P>
inline P* at(const void* base, size_t off) {
    return reinterpret_cast<P*>(reinterpret_cast<uintptr_t>(base) + off);
}

// K splits of the x-projection: about two workgroups per CU, each with at least 512 K
// K splits of the x-projection: about 512 workgroups with at least 512 channels each; a grid of
// a few tiles instead takes one 128-channel chunk per workgroup (at most 64 splits), since each
// of a workgroup's K steps waits for its projection rows and so few workgroups cannot hide it
int xproj_ksplit(int T, int d_in, int ncols_pad) {
    if (T <= 0 || ncols_pad <= 0) return 1;
    const int tiles = (T + 127) / 128 * ((ncols_pad + 319) / 320);
    int ks = tiles <= 4 ? std::min(d_in / 128, 64) : std::min((512 + tiles - 1) / tiles, std::max(1, d_in / 512));
    return std::max(ks, 1);
}

int ensure_attributes() {
    QE_TRY_HIP(skinny_set_attributes());
    return QE_OK;
}

}  // namespace

namespace qe {
constexpr int kSkinnyMaxT = 16;  // token counts served by the weight-streaming kernels
// Size of the per-GPU scratch array of qe_linear_forward_noalloc: enough for the decode and
// few-token calls of every linear up to the 72B MLP widths (its workspace at 16 tokens and
// 29568 input channels is about 15 MB).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
int noalloc_scratch(void** out);

// Prefill prologue in two reads of x (route pass, then expert-sorted quantization), for
// bf16 activations; the workspace is sized for it whatever the activation type
bool two_pass_sized(const qe_linear* lin, int T) { return lin->a_bits != 16 && T > kSkinnyMaxT; }
// few-token prefill with bf16 x: the one-launch prologue where its shape limits allow
bool row_prologue(const qe_linear* lin, int T, int x_dtype) {
    return two_pass_sized(lin, T) && x_dtype == QE_BF16 &&
           row_prologue_ok(T, lin->d_in, rank_pad(lin->r_shared), lin->n_routed,
                           lin->n_routed > 0 ? rank_pad(lin->r_routed) : 0);
}
}  // namespace qe

namespace qe {

PrepLayout prep_layout(const qe_linear* lin) {
    PrepLayout L{};
    const size_t d_in = lin->d_in, d_out = lin->d_out;
    L.rs_pad = rank_pad(lin->r_shared);
    L.rr_pad = lin->n_routed > 0 ? rank_pad(lin->r_routed) : 0;
    L.has_smooth = lin->a_bits != 16;
    // Mt rows: [A_s^T (rs_pad) ; R^T (padded to 16) ; A_1^T .. A_N^T (rr_pad each)], so
    // the shared expert and the router form one leading block of at most 80 rows
    const int router_pad = lin->n_routed > 0 ? (lin->n_routed + 15) / 16 * 16 : 0;
    L.col_se = L.rs_pad > 0 ? 0 : -1;
    L.col_router = lin->n_routed > 0 ? L.rs_pad : -1;
    L.col_re = lin->n_routed > 0 ? L.rs_pad + router_pad : -1;
    L.n_lead = L.rs_pad + router_pad;
    L.n_cols = L.n_lead + lin->n_routed * L.rr_pad;
    L.n_cols_pad = (L.n_cols + 15) / 16 * 16;
    size_t off = 0;
    L.w_tiled = off;
    L.w_tiled_bytes = lin->w_bits == 4 ? d_out * d_in / 2 : d_out * d_in * 3 / 8;
    off = align256(off + L.w_tiled_bytes);
    L.w_scale = off;
    off = align256(off + d_out * 4);
    L.smooth = off;
    off = align256(off + (L.has_smooth ? d_in * 4 : 0));
    L.inv_smooth = off;
    off = align256(off + (L.has_smooth ? d_in * 4 : 0));
    L.mt = off;
    off = align256(off + (size_t)L.n_cols_pad * d_in * 2);
    L.bt_s = off;
    off = align256(off + d_out * L.rs_pad * 2);
    L.bt_r = off;
    off = align256(off + (size_t)lin->n_routed * d_out * L.rr_pad * 2);
    L.total = off;
    return L;
}

WsLayout ws_layout(const qe_linear* lin, int T) {
    WsLayout W{};
    const PrepLayout P = prep_layout(lin);
    const size_t t = T > 0 ? T : 0;
    W.xproj_ksplit = xproj_ksplit(T, lin->d_in, P.n_cols_pad);
    W.skinny_ksplit = lin->a_bits != 16 ? 0
                      : T <= kSkinnyMaxT ? skinny_ksplit(lin->d_in, lin->d_out)
                                         : gemm_a16_ksplit(T, lin->d_in, lin->d_out, lin->w_bits);
    const bool fused_decode = T <= kSkinnyMaxT && (lin->a_bits == 16 || lin->w_bits == 4);
    const DecodePlan D = fused_decode ? decode_plan(lin->d_in, lin->d_out, lin->w_bits, P.n_cols_pad, T) : DecodePlan{};
    size_t off = 0;
    W.codes = off;
    off = align256(off + (lin->a_bits == 16 ? 0 : t * lin->d_in));
    W.s_x = off;
    off = align256(off + t * 4);
    W.part = off;
    const int xks = std::max({W.xproj_ksplit, T <= kSkinnyMaxT ? skinny_ksplit_proj(lin->d_in) : 1, D.ks_p});
    const bool two_pass = two_pass_sized(lin, T);
    W.rp_ksplit = two_pass ? route_pass_ksplit(T, lin->d_in) : 0;
    W.eq_ksplit = two_pass ? expert_quant_ksplit(T, lin->d_in) : 0;
    off = align256(off + std::max((size_t)xks * t * P.n_cols_pad, (size_t)W.rp_ksplit * t * P.n_lead) * 4);
    W.amax = off;
    off = align256(off + (size_t)W.rp_ksplit * t * 4);
    W.vpart = off;
    off = align256(off + (W.eq_ksplit > 1 ? (size_t)W.eq_ksplit * t * P.rr_pad * 4 : 0));

    W.scores = off;
    off = align256(off + t * std::max(lin->n_routed, 1) * 4);
    W.expert = off;
    off = align256(off + t * 4);
    W.counts = off;
    off = align256(off + 32 * 4);
    W.offsets = off;
    off = align256(off + 32 * 4);
    W.perm = off;
    off = align256(off + t * 4);
    W.u = off;
    off = align256(off + t * P.rs_pad * 2);
    W.v = off;
    off = align256(off + t * P.rr_pad * 2);
    W.gemm_ksplit = lin->a_bits != 16 ? gemm_ksplit(T, lin->d_in, lin->d_out) : 1;
    W.skinny = off;
    off = align256(off + (size_t)std::max({W.skinny_ksplit, D.ks_m, W.gemm_ksplit > 1 ? W.gemm_ksplit : 0}) * t *
                             lin->d_out * 4);
    W.total = off;
    return W;
}

}  // namespace qe

// ------------------------------------------------------------ allocation-free forward
// The workspace of qe_linear_forward_noalloc: one file-scope device array per GPU, held until
// the process ends.  Host code never passes the array's name to a kernel (on the host it only
// names a stand-in): its device address is taken per device with hipGetSymbolAddress on the
// first call on that device, with that device current, and only that address is used.
static __device__ __align__(256) uint8_t scratch[qe::kNoAllocScratchBytes];

namespace qe {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of the current device's scratch array (looked up once per device).
int noalloc_scratch(void** out) {
    int dev = 0;
    QE_TRY_HIP(hipGetDevice(&dev));
    QE_CHECK(dev >= 0 && dev < kMaxDevices, QE_ERR_UNSUPPORTED);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        QE_TRY_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
        QE_CHECK(ptr != nullptr, QE_ERR_HIP);
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return QE_OK;
}
}  // namespace qe

// ======================================================================= ABI
extern "C" {

const char* qe_status_string(int status) {
    switch (status) {
        case QE_OK: return "QE_OK";
        case QE_ERR_INVALID_ARG: return "QE_ERR_INVALID_ARG";
        case QE_ERR_UNSUPPORTED: return "QE_ERR_UNSUPPORTED";
        case QE_ERR_ALIGNMENT: return "QE_ERR_ALIGNMENT";
        case QE_ERR_WORKSPACE: return "QE_ERR_WORKSPACE";
        case QE_ERR_HIP: return "QE_ERR_HIP";
        default: return "QE_UNKNOWN_STATUS";
    }
}

int qe_last_hip_error(void) { return g_last_hip_error; }

const char* qe_version(void) { return "libqe 0.1 (gfx950)"; }

// ------------------------------------------------------------------ weights
int qe_pack_weights(const float* W_f, const float* s, int32_t d_out, int32_t d_in, int32_t w_bits, void* packed,
                    float* w_scale) {
    QE_CHECK(W_f && packed && w_scale, QE_ERR_INVALID_ARG);
    QE_CHECK(d_out > 0 && d_in > 0, QE_ERR_INVALID_ARG);
    QE_CHECK(w_bits == 3 || w_bits == 4, QE_ERR_INVALID_ARG);
    QE_CHECK(w_bits == 4 ? d_in % 2 == 0 : d_in % 32 == 0, QE_ERR_UNSUPPORTED);
    const float qmax = w_bits == 4 ? 7.0f : 3.0f;
    const size_t row_bytes = w_bits == 4 ? (size_t)d_in / 2 : (size_t)d_in / 32 * 12;
    auto work = [&](int r0, int r1) {
        std::vector<float> wp(d_in);
        std::vector<int> q(d_in);
        for (int i = r0; i < r1; ++i) {
            const float* row = W_f + (size_t)i * d_in;
            float amax = 0.0f;
            for (int j = 0; j < d_in; ++j) {
                float v = s ? row[j] * s[j] : row[j];
                wp[j] = v;
                amax = std::max(amax, std::fabs(v));
            }
            const float sw = amax / qmax;
            w_scale[i] = sw;
            for (int j = 0; j < d_in; ++j) {
                float c = 0.0f;
                if (amax > 0.0f) c = std::min(std::max(std::nearbyint(wp[j] / sw), -qmax), qmax);
                q[j] = (int)c;
            }
            uint8_t* out = reinterpret_cast<uint8_t*>(packed) + (size_t)i * row_bytes;
            if (w_bits == 4) {
                for (int m = 0; m < d_in / 2; ++m)
                    out[m] = (uint8_t)((q[2 * m] & 0xF) | ((q[2 * m + 1] & 0xF) << 4));
            } else {
                for (int g = 0; g < d_in / 32; ++g) {
                    uint32_t w3[3] = {0, 0, 0};
                    for (int c = 0; c < 32; ++c) {
                        const uint32_t code = (uint32_t)q[g * 32 + c] & 7u;
                        const int bit = 3 * c, wi = bit >> 5, off = bit & 31;
                        w3[wi] |= code << off;
                        if (off > 29) w3[wi + 1] |= code >> (32 - off);
                    }
                    std::memcpy(out + (size_t)g * 12, w3, 12);
                }
            }
        }
    };
    const int hw = std::max(1u, std::min(32u, std::thread::hardware_concurrency()));
    const int nthreads = std::min<long>(hw, std::max<long>(1, (long)d_out * d_in / (1 << 20)));
    if (nthreads <= 1) {
        work(0, d_out);
    } else {
        std::vector<std::thread> th;
        for (int k = 0; k < nthreads; ++k) {
            const int r0 = (int)((long)d_out * k / nthreads), r1 = (int)((long)d_out * (k + 1) / nthreads);
            th.emplace_back(work, r0, r1);
        }
        for (auto& t : th) t.join();
    }
    return QE_OK;
}

size_t qe_prepared_bytes(const qe_linear* lin) {
    if (validate_linear(lin) != QE_OK) return 0;
    return prep_layout(lin).total;
}

int qe_prepare(const qe_linear* lin, const void* w_packed, const float* w_scale, const float* smooth,
               const uint16_t* A_s, const uint16_t* B_s, const uint16_t* A_r, const uint16_t* B_r, const uint16_t* R,
               void* prep, void* stream) {
    int st = validate_linear(lin);
    if (st) return st;
    QE_CHECK(w_packed && w_scale && prep, QE_ERR_INVALID_ARG);
    QE_CHECK((lin->r_shared > 0) == (A_s != nullptr) && (lin->r_shared > 0) == (B_s != nullptr), QE_ERR_INVALID_ARG);
    QE_CHECK((lin->n_routed > 0) == (A_r != nullptr) && (lin->n_routed > 0) == (B_r != nullptr) &&
                 (lin->n_routed > 0) == (R != nullptr),
             QE_ERR_INVALID_ARG);
    QE_CHECK(!(lin->a_bits == 16 && smooth != nullptr), QE_ERR_INVALID_ARG);
    for (const void* p : {w_packed, (const void*)w_scale, (const void*)prep})
        QE_CHECK(aligned16(p), QE_ERR_ALIGNMENT);
    const PrepLayout L = prep_layout(lin);
    hipStream_t s = S(stream);
    const int d_in = lin->d_in, d_out = lin->d_out;
    if (lin->w_bits == 4) {
        QE_TRY_HIP(launch_prep_w4(reinterpret_cast<const uint8_t*>(w_packed), d_out, d_in, at<uint8_t>(prep, L.w_tiled), s));
    } else {
        QE_TRY_HIP(launch_prep_w3(reinterpret_cast<const uint32_t*>(w_packed), d_out, d_in, at<uint32_t>(prep, L.w_tiled), s));
    }
    QE_TRY_HIP(hipMemcpyAsync(at<void>(prep, L.w_scale), w_scale, (size_t)d_out * 4, hipMemcpyDeviceToDevice, s));
    if (L.has_smooth)
        QE_TRY_HIP(launch_prep_smooth(smooth, d_in, at<float>(prep, L.smooth), at<float>(prep, L.inv_smooth), s));
    // Mt: [A_s^T ; R^T ; A_1^T .. A_N^T], zero rows in the padding
    uint16_t* mt = at<uint16_t>(prep, L.mt);
    QE_TRY_HIP(launch_fill_zero(mt, (size_t)L.n_cols_pad * d_in * 2, s));
    if (L.rs_pad > 0) QE_TRY_HIP(launch_prep_transpose(A_s, d_in, lin->r_shared, mt + (size_t)L.col_se * d_in, d_in, L.rs_pad, s));
    for (int e = 0; e < lin->n_routed; ++e) {
        QE_TRY_HIP(launch_prep_transpose(A_r + (size_t)e * d_in * lin->r_routed, d_in, lin->r_routed,
                                         mt + (size_t)(L.col_re + e * L.rr_pad) * d_in, d_in, L.rr_pad, s));
    }
    if (lin->n_routed > 0)
        QE_TRY_HIP(launch_prep_transpose(R, d_in, lin->n_routed, mt + (size_t)L.col_router * d_in, d_in, lin->n_routed, s));
    // Bt_s [d_out][rs_pad], Bt_r [N][d_out][rr_pad]
    if (L.rs_pad > 0) QE_TRY_HIP(launch_prep_transpose(B_s, lin->r_shared, d_out, at<uint16_t>(prep, L.bt_s), L.rs_pad, d_out, s));
    for (int e = 0; e < lin->n_routed; ++e) {
        QE_TRY_HIP(launch_prep_transpose(B_r + (size_t)e * lin->r_routed * d_out, lin->r_routed, d_out,
                                         at<uint16_t>(prep, L.bt_r) + (size_t)e * d_out * L.rr_pad, L.rr_pad, d_out, s));
    }
    return QE_OK;
}

size_t qe_workspace_bytes(const qe_linear* lin, int32_t T) {
    if (validate_linear(lin) != QE_OK || T < 0) return 0;
    return ws_layout(lin, T).total;
}

// ------------------------------------------------------------------ a1
int qe_quant_act(const void* x, int32_t x_dtype, const float* smooth, int32_t T, int32_t d_in, int32_t a_bits,
                 int8_t* codes, float* s_x, void* stream) {
    QE_CHECK(T >= 0 && d_in > 0, QE_ERR_INVALID_ARG);
    QE_CHECK(a_bits == 6 || a_bits == 8, QE_ERR_INVALID_ARG);
    QE_CHECK(x_dtype == QE_F32 || x_dtype == QE_BF16, QE_ERR_INVALID_ARG);
    QE_CHECK(d_in % 8 == 0 && d_in <= 32768, QE_ERR_UNSUPPORTED);
    if (T == 0) return QE_OK;
    QE_CHECK(x && codes && s_x, QE_ERR_INVALID_ARG);
    for (const void* p : {x, (const void*)codes, (const void*)s_x}) QE_CHECK(aligned16(p), QE_ERR_ALIGNMENT);
    if (smooth) QE_CHECK(aligned16(smooth), QE_ERR_ALIGNMENT);
    QE_TRY_HIP(launch_quant_act(x, x_dtype, smooth, nullptr, T, d_in, a_bits, codes, s_x, S(stream)));
    return QE_OK;
}

// Projection of x onto the columns [c0, c0 + nc) of the prepared Mt, then the
// per-token reduction / routing.  Internal helper for route / adapter inputs / forward.
// Split-K partial sums of x onto the projection columns [c0, c0 + nc) (padded to nc_pad); *ks
// receives the split count the finish kernel needs.
static int xpass_partials(const qe_linear* lin, const void* x, int x_dtype, int T, int c0, int nc, int nc_pad,
                          float* part, void* ws, hipStream_t s, int* ks) {
    const PrepLayout P = prep_layout(lin);
    const WsLayout W = ws_layout(lin, T);
    const uint16_t* mt = at<const uint16_t>(lin->prep, P.mt);
    if (T <= kSkinnyMaxT) {  // few tokens: stream the projection matrix like decode weights
        int st = ensure_attributes();
        if (st) return st;
        *ks = skinny_ksplit_proj(lin->d_in);
        QE_TRY_HIP(launch_skinny(x, x_dtype, T, lin->d_in, nc_pad, 16, mt + (size_t)c0 * lin->d_in, *ks, part, nc_pad, s));
    } else {
        *ks = std::min(W.xproj_ksplit, xproj_ksplit(T, lin->d_in, nc_pad));
        QE_TRY_HIP(launch_xproj(x, x_dtype, T, lin->d_in, mt, c0, nc, nc_pad, *ks, part, s));
    }
    (void)ws;
    return QE_OK;
}

static int run_xpass(const qe_linear* lin, const void* x, int x_dtype, int T, bool want_se, bool want_re,
                     bool do_route, const int32_t* expert_in, float* scores, int32_t* expert_out, uint16_t* u,
                     uint16_t* v, void* ws, hipStream_t s, int32_t* expert2_out = nullptr) {
    const PrepLayout P = prep_layout(lin);
    const WsLayout W = ws_layout(lin, T);
    int c0 = P.n_cols, c1 = 0;
    auto include = [&](int beg, int n) {
        if (beg < 0 || n <= 0) return;
        c0 = std::min(c0, beg);
        c1 = std::max(c1, beg + n);
    };
    if (want_se) include(P.col_se, P.rs_pad);
    if (want_re) include(P.col_re, lin->n_routed * P.rr_pad);
    if (do_route) include(P.col_router, lin->n_routed);
    if (c1 <= c0) return QE_OK;
    const int nc = c1 - c0, nc_pad = (nc + 15) / 16 * 16;
    float* part = at<float>(ws, W.part);
    int ks = 0;
    int st = xpass_partials(lin, x, x_dtype, T, c0, nc, nc_pad, part, ws, s, &ks);
    if (st) return st;
    QE_TRY_HIP(launch_xproj_finish(part, ks, T, nc_pad, c0, want_se ? P.col_se : -1, lin->r_shared, P.rs_pad,
                                   want_re ? P.col_re : -1, lin->n_routed, lin->r_routed, P.rr_pad,
                                   do_route ? P.col_router : -1, expert_in, scores, expert_out, want_se ? u : nullptr,
                                   want_re ? v : nullptr, s, do_route ? expert2_out : nullptr));
    return QE_OK;
}

// ------------------------------------------------------------------ a5
int qe_route(const qe_linear* lin, const void* x, int32_t x_dtype, int32_t T, float* scores, int32_t* expert,
             int32_t* counts, int32_t* offsets, int32_t* perm, void* ws, size_t ws_bytes, void* stream) {
    int st = validate_forward_common(lin, T, x_dtype, x, ws, ws_bytes);
    if (st) return st;
    QE_CHECK(lin->n_routed > 0, QE_ERR_INVALID_ARG);
    if (T == 0) return QE_OK;
    QE_CHECK(x && expert && counts && offsets && perm, QE_ERR_INVALID_ARG);
    hipStream_t s = S(stream);
    st = run_xpass(lin, x, x_dtype, T, false, false, true, nullptr, scores, expert, nullptr, nullptr, ws, s);
    if (st) return st;
    QE_TRY_HIP(launch_bucket(expert, T, lin->n_routed, counts, offsets, perm, s));
    return QE_OK;
}

// ------------------------------------------------------------------ a4/a6 inputs
int qe_adapter_inputs(const qe_linear* lin, const void* x, int32_t x_dtype, int32_t T, const int32_t* expert,
                      uint16_t* u, uint16_t* v, void* ws, size_t ws_bytes, void* stream) {
    int st = validate_forward_common(lin, T, x_dtype, x, ws, ws_bytes);
    if (st) return st;
    QE_CHECK((lin->r_shared > 0) == (u != nullptr), QE_ERR_INVALID_ARG);
    QE_CHECK((lin->n_routed > 0) == (v != nullptr) && (lin->n_routed > 0) == (expert != nullptr), QE_ERR_INVALID_ARG);
    if (T == 0) return QE_OK;
    QE_CHECK(x != nullptr, QE_ERR_INVALID_ARG);
    return run_xpass(lin, x, x_dtype, T, u != nullptr, v != nullptr, false, expert, nullptr, nullptr, u, v, ws, S(stream));
}

// ------------------------------------------------------------------ a3 / a7
static int run_gemm(const qe_linear* lin, const int8_t* codes, const float* s_x, const void* x, int x_dtype, int T,
                    const uint16_t* u, const uint16_t* v, const int32_t* expert, const int32_t* perm, float* y,
                    int32_t* acc_debug, void* ws, hipStream_t s) {
    const PrepLayout P = prep_layout(lin);
    const uint16_t* bt_s = P.rs_pad > 0 ? at<const uint16_t>(lin->prep, P.bt_s) : nullptr;
    const uint16_t* bt_r = P.rr_pad > 0 ? at<const uint16_t>(lin->prep, P.bt_r) : nullptr;
    const float* w_scale = at<const float>(lin->prep, P.w_scale);
    const bool y_bf16 = lin->y_dtype == QE_BF16;
    if (!bt_s) u = nullptr;
    if (!bt_r) v = nullptr;
    if (lin->a_bits == 16) {
        const WsLayout W = ws_layout(lin, T);
        float* part = at<float>(ws, W.skinny);
        int st = ensure_attributes();
        if (st) return st;
        if (T > kSkinnyMaxT) {  // every weight fragment used for 64 or 128 tokens
            QE_TRY_HIP(launch_gemm_a16(x, x_dtype, T, lin->d_in, lin->d_out, lin->w_bits,
                                       at<const void>(lin->prep, P.w_tiled), W.skinny_ksplit, part, w_scale, u, bt_s,
                                       P.rs_pad, v, expert, bt_r, P.rr_pad, lin->n_routed, y, y_bf16, s));
            return QE_OK;
        }
        // weight streaming, the tokens as one MFMA block
        QE_TRY_HIP(launch_skinny(x, x_dtype, T, lin->d_in, lin->d_out, lin->w_bits, at<const void>(lin->prep, P.w_tiled),
                                 W.skinny_ksplit, part, lin->d_out, s));
        QE_TRY_HIP(launch_skinny_finish(part, W.skinny_ksplit, T, lin->d_out, w_scale, u, bt_s, P.rs_pad, v, expert,
                                        bt_r, P.rr_pad, y, y_bf16, s));
    } else {
        const WsLayout W = ws_layout(lin, T);
        const int ks = acc_debug ? 1 : W.gemm_ksplit;
        QE_TRY_HIP(launch_gemm_w4(codes, s_x, at<const uint8_t>(lin->prep, P.w_tiled), w_scale, T, lin->d_in,
                                  lin->d_out, u, bt_s, P.rs_pad, v, expert, bt_r, P.rr_pad, lin->n_routed, perm, y,
                                  acc_debug, ks, ks > 1 ? at<int32_t>(ws, W.skinny) : nullptr, y_bf16, s));
    }
    return QE_OK;
}

int qe_wq_gemm(const qe_linear* lin, const int8_t* codes, const float* s_x, const void* x, int32_t x_dtype, int32_t T,
               const uint16_t* u, const uint16_t* v, const int32_t* expert, const int32_t* perm, float* y,
               int32_t* acc_debug, void* ws, size_t ws_bytes, void* stream) {
    int st = validate_forward_common(lin, T, x_dtype, x, ws, ws_bytes);
    if (st) return st;
    if (T == 0) return QE_OK;
    QE_CHECK(y != nullptr, QE_ERR_INVALID_ARG);
    QE_CHECK(aligned16(y), QE_ERR_ALIGNMENT);
    if (lin->a_bits == 16) {
        QE_CHECK(x != nullptr && acc_debug == nullptr, QE_ERR_INVALID_ARG);
    } else {
        QE_CHECK(codes && s_x, QE_ERR_INVALID_ARG);
        QE_CHECK(aligned16(codes), QE_ERR_ALIGNMENT);
    }
    QE_CHECK((v == nullptr) == (expert == nullptr), QE_ERR_INVALID_ARG);
    return run_gemm(lin, codes, s_x, x, x_dtype, T, u, v, expert, lin->a_bits == 16 ? nullptr : perm, y, acc_debug, ws,
                    S(stream));
}

// ------------------------------------------------------------------ a6 unfused
int qe_routed_lora(const qe_linear* lin, const void* x, int32_t x_dtype, int32_t T, const int32_t* expert,
                   const int32_t* offsets, const int32_t* perm, float* y, void* ws, size_t ws_bytes, void* stream) {
    int st = validate_forward_common(lin, T, x_dtype, x, ws, ws_bytes);
    if (st) return st;
    QE_CHECK(lin->n_routed > 0, QE_ERR_INVALID_ARG);
    QE_CHECK(T <= 65535, QE_ERR_UNSUPPORTED);
    QE_CHECK(lin->y_dtype == QE_F32, QE_ERR_UNSUPPORTED);  // adds into y in place
    if (T == 0) return QE_OK;
    QE_CHECK(x && expert && offsets && perm && y, QE_ERR_INVALID_ARG);
    const PrepLayout P = prep_layout(lin);
    const WsLayout W = ws_layout(lin, T);
    hipStream_t s = S(stream);
    uint16_t* v = at<uint16_t>(ws, W.v);
    st = run_xpass(lin, x, x_dtype, T, false, true, false, expert, nullptr, nullptr, nullptr, v, ws, s);
    if (st) return st;
    QE_TRY_HIP(launch_routed_lora(v, P.rr_pad, offsets, perm, lin->n_routed, at<const uint16_t>(lin->prep, P.bt_r), T,
                                  lin->d_out, y, s));
    return QE_OK;
}

// ------------------------------------------------------------------ composite
// The two-pass prologue after its route pass (whose partials are in ws): route finish, then the
// expert-sorted quantization pass.
static int run_prologue_rest(const qe_linear* lin, const void* x, int T, int8_t* codes, float* s_x, uint16_t* u,
                             uint16_t* v, int32_t* expert, int32_t* perm, void* ws, hipStream_t s, bool keep_order,
                             int32_t* expert2 = nullptr) {
    const PrepLayout P = prep_layout(lin);
    const WsLayout W = ws_layout(lin, T);
    const bool route = lin->n_routed > 0;
    const float* smooth = at<const float>(lin->prep, P.smooth);
    const float* inv_smooth = at<const float>(lin->prep, P.inv_smooth);
    const uint16_t* mt = at<const uint16_t>(lin->prep, P.mt);
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
    QE_TRY_HIP(launch_route_finish(at<const float>(ws, W.part), at<const float>(ws, W.amax), W.rp_ksplit, T,
                                       P.n_lead, lin->r_shared, P.rs_pad, P.col_router, lin->n_routed, lin->a_bits,
                                       route ? expert : nullptr, u, s_x, s, route ? expert2 : nullptr));
        QE_TRY_HIP(launch_expert_quant(xb, T, lin->d_in, smooth, inv_smooth, s_x, lin->a_bits,
                                       route ? expert : nullptr, lin->n_routed,
                                       route ? mt + (size_t)P.col_re * lin->d_in : nullptr, P.rr_pad, lin->r_routed,
                                       W.eq_ksplit, route ? (perm ? perm : at<int32_t>(ws, W.perm)) : nullptr,
                                       at<float>(ws, W.vpart), codes, route ? v : nullptr, keep_order, s));
    return QE_OK;
}

// keep_order: few tokens may stay in token order in the two-pass prologue (perm is then not
// written; the caller passes perm == NULL)
// expert2 (top-2 routing, optional): also the second expert of every token
static int run_prologue(const qe_linear* lin, const void* x, int x_dtype, int T, int8_t* codes, float* s_x,
                        uint16_t* u, uint16_t* v, int32_t* expert, int32_t* perm, void* ws, hipStream_t s,
                        bool keep_order = false, int32_t* expert2 = nullptr) {
    const PrepLayout P = prep_layout(lin);
    const WsLayout W = ws_layout(lin, T);
    const bool route = lin->n_routed > 0;
    if (row_prologue(lin, T, x_dtype) && !expert2) {
        // few tokens: one launch, everything in token order; the expert order the GEMM's tiles
        // walk (when it is asked for) comes from the bucketing kernel
        QE_TRY_HIP(launch_row_prologue(reinterpret_cast<const uint16_t*>(x), T, lin->d_in,
                                       at<const float>(lin->prep, P.smooth), at<const float>(lin->prep, P.inv_smooth),
                                       lin->a_bits, at<const uint16_t>(lin->prep, P.mt), lin->r_shared, P.rs_pad,
                                       P.col_router, lin->n_routed, P.col_re, lin->r_routed, P.rr_pad, codes, s_x,
                                       P.rs_pad > 0 ? u : nullptr, route ? expert : nullptr, route ? v : nullptr, s));
        if (route && perm)
            QE_TRY_HIP(launch_bucket(expert, T, lin->n_routed, at<int32_t>(ws, W.counts), at<int32_t>(ws, W.offsets),
                                     perm, s));
        return QE_OK;
    }
    if (two_pass_sized(lin, T) && x_dtype == QE_BF16) {
        QE_TRY_HIP(launch_route_pass(reinterpret_cast<const uint16_t*>(x), T, lin->d_in,
                                     at<const uint16_t>(lin->prep, P.mt), P.n_lead, at<const float>(lin->prep, P.smooth),
                                     at<const float>(lin->prep, P.inv_smooth), W.rp_ksplit, at<float>(ws, W.part),
                                     at<float>(ws, W.amax), s));
        return run_prologue_rest(lin, x, T, codes, s_x, u, v, expert, perm, ws, s, keep_order, expert2);
    }
    int st = run_xpass(lin, x, x_dtype, T, u != nullptr, route, route, nullptr, nullptr, route ? expert : nullptr, u,
                       v, ws, s, route ? expert2 : nullptr);
    if (st) return st;
    if (route && perm)  // tokens grouped by routed expert, for the GEMM's tile order
        QE_TRY_HIP(launch_bucket(expert, T, lin->n_routed, at<int32_t>(ws, W.counts), at<int32_t>(ws, W.offsets), perm, s));
    if (lin->a_bits != 16)
        QE_TRY_HIP(launch_quant_act(x, x_dtype, at<const float>(lin->prep, P.smooth),
                                    at<const float>(lin->prep, P.inv_smooth), T, lin->d_in, lin->a_bits, codes, s_x, s));
    return QE_OK;
}

int qe_linear_prologue(const qe_linear* lin, const void* x, int32_t x_dtype, int32_t T, int8_t* codes, float* s_x,
                       uint16_t* u, uint16_t* v, int32_t* expert, int32_t* perm, void* ws, size_t ws_bytes,
                       void* stream) {
    int st = validate_forward_common(lin, T, x_dtype, x, ws, ws_bytes);
    if (st) return st;
    if (T == 0) return QE_OK;
    QE_CHECK(x != nullptr, QE_ERR_INVALID_ARG);
    QE_CHECK(lin->a_bits == 16 ? (codes == nullptr && s_x == nullptr) : (codes && s_x), QE_ERR_INVALID_ARG);
    QE_CHECK((lin->r_shared > 0) == (u != nullptr), QE_ERR_INVALID_ARG);
    QE_CHECK((lin->n_routed > 0) == (v != nullptr) && (lin->n_routed > 0) == (expert != nullptr), QE_ERR_INVALID_ARG);
    QE_CHECK(!perm || lin->n_routed > 0, QE_ERR_INVALID_ARG);
    if (codes) QE_CHECK(aligned16(codes), QE_ERR_ALIGNMENT);
    return run_prologue(lin, x, x_dtype, T, codes, s_x, u, v, expert, perm, ws, S(stream));
}

int qe_linear_forward(const qe_linear* lin, const void* x, int32_t x_dtype, int32_t T, float* y, int32_t* expert_out,
                      void* ws, size_t ws_bytes, void* stream) {
    int st = validate_forward_common(lin, T, x_dtype, x, ws, ws_bytes);
    if (st) return st;
    if (T == 0) return QE_OK;
    QE_CHECK(x && y, QE_ERR_INVALID_ARG);
    QE_CHECK(aligned16(y), QE_ERR_ALIGNMENT);
    const PrepLayout P = prep_layout(lin);
    const WsLayout W = ws_layout(lin, T);
    hipStream_t s = S(stream);
    const bool route = lin->n_routed > 0;
    int32_t* expert = route ? (expert_out ? expert_out : at<int32_t>(ws, W.expert)) : nullptr;
    uint16_t* u = P.rs_pad > 0 ? at<uint16_t>(ws, W.u) : nullptr;
    uint16_t* v = route ? at<uint16_t>(ws, W.v) : nullptr;
    if (T <= kSkinnyMaxT && (lin->a_bits == 16 || lin->w_bits == 4)) {
        // decode: one launch streams the projection matrix and the packed weights, one finishes;
        // with quantized activations the codes are made first and the weights meet them on the
        // int8 matrix cores
        int e = ensure_attributes();
        if (e) return e;
        const DecodePlan D = decode_plan(lin->d_in, lin->d_out, lin->w_bits, P.n_cols_pad, T);
        float* part_m = at<float>(ws, W.skinny);
        float* part_p = at<float>(ws, W.part);
        int8_t* dcodes = nullptr;
        float* ds_x = nullptr;
        if (lin->a_bits != 16) {
            dcodes = at<int8_t>(ws, W.codes);
            ds_x = at<float>(ws, W.s_x);
            QE_TRY_HIP(launch_quant_act(x, x_dtype, at<const float>(lin->prep, P.smooth),
                                        at<const float>(lin->prep, P.inv_smooth), T, lin->d_in, lin->a_bits, dcodes,
                                        ds_x, s));
        }
        QE_TRY_HIP(launch_decode_gemv(x, x_dtype, dcodes, T, lin->d_in, lin->d_out, lin->w_bits,
                                      at<const void>(lin->prep, P.w_tiled), D, part_m,
                                      at<const uint16_t>(lin->prep, P.mt), P.n_cols_pad, part_p, s));
        QE_TRY_HIP(launch_decode_finish(part_m, ds_x, D.ks_m, T, lin->d_out, at<const float>(lin->prep, P.w_scale), part_p,
                                        D.ks_p, P.n_cols_pad, P.col_se, lin->r_shared, P.rs_pad, P.col_re,
                                        lin->n_routed, lin->r_routed, P.rr_pad, P.col_router,
                                        P.rs_pad > 0 ? at<const uint16_t>(lin->prep, P.bt_s) : nullptr,
                                        P.rr_pad > 0 ? at<const uint16_t>(lin->prep, P.bt_r) : nullptr,
                                        route ? expert : nullptr, y, lin->y_dtype == QE_BF16, s));
        return QE_OK;
    }
    int8_t* codes = lin->a_bits != 16 ? at<int8_t>(ws, W.codes) : nullptr;
    float* s_x = lin->a_bits != 16 ? at<float>(ws, W.s_x) : nullptr;
    // the GEMM visits the tokens grouped by expert, except for few tokens whose main product
    // is split over K (its finish handles every token's expert alike): then the two-pass
    // prologue keeps token order and skips the bucketing
    const bool keep_order = two_pass_sized(lin, T) && x_dtype == QE_BF16 && expert_quant_few(T) && W.gemm_ksplit > 1;
    int32_t* perm = (route && lin->a_bits != 16 && !keep_order) ? at<int32_t>(ws, W.perm) : nullptr;
    st = run_prologue(lin, x, x_dtype, T, codes, s_x, u, v, expert, perm, ws, s, keep_order);
    if (st) return st;
    return run_gemm(lin, codes, s_x, x, x_dtype, T, u, v, expert, perm, y, nullptr, ws, s);
}

// ------------------------------------------------------------------ linears sharing one input
// Whether a group of linears takes the grouped route pass: 2..3 linears on the same bf16 x, all
// on the two-pass prefill prologue, with the same d_in and at most 48 projected columns each.
static bool group_route_pass(const qe_linear* const* lins, int n, int x_dtype, int T) {
    if (n < 2 || n > RG_MAX || x_dtype != QE_BF16) return false;
    for (int i = 0; i < n; ++i) {
        // few tokens: each linear's one-launch prologue (bit-identical to a linear's own call)
        if (!two_pass_sized(lins[i], T) || row_prologue(lins[i], T, x_dtype) || lins[i]->d_in != lins[0]->d_in)
            return false;
        const int nl = prep_layout(lins[i]).n_lead;
        if (nl < 16 || nl > 48) return false;
    }
    return true;
}

static int validate_group(const qe_linear* const* lins, int32_t n, int32_t T, int32_t x_dtype, const void* x,
                          void* const* ws, const size_t* ws_bytes) {
    QE_CHECK(lins && n >= 1 && n <= RG_MAX && ws && ws_bytes, QE_ERR_INVALID_ARG);
    for (int i = 0; i < n; ++i) {
        int st = validate_forward_common(lins[i], T, x_dtype, x, ws[i], ws_bytes[i]);
        if (st) return st;
        QE_CHECK(lins[i]->d_in == lins[0]->d_in, QE_ERR_INVALID_ARG);
    }
    return QE_OK;
}

// One read of x for the route passes of the group: each linear's partials land where its own
// route pass would put them (its workspace), then each linear's route finish and quantization.
static int run_group_prologue(const qe_linear* const* lins, int n, const void* x, int x_dtype, int T,
                              int8_t* const* codes, float* const* s_x, uint16_t* const* u, uint16_t* const* v,
                              int32_t* const* expert, int32_t* const* perm, void* const* ws, hipStream_t s,
                              const bool* keep_order) {
    if (!group_route_pass(lins, n, x_dtype, T)) {
        for (int i = 0; i < n; ++i) {
            int st = run_prologue(lins[i], x, x_dtype, T, codes[i], s_x[i], u[i], v[i], expert[i], perm[i], ws[i], s,
                                  keep_order ? keep_order[i] : false);
            if (st) return st;
        }
        return QE_OK;
    }
    RouteGroup G{};
    int ks = 0;
    for (int i = 0; i < n; ++i) {
        const PrepLayout P = prep_layout(lins[i]);
        const WsLayout W = ws_layout(lins[i], T);
        G.mt[i] = at<const uint16_t>(lins[i]->prep, P.mt);
        G.smooth[i] = at<const float>(lins[i]->prep, P.smooth);
        G.inv_smooth[i] = at<const float>(lins[i]->prep, P.inv_smooth);
        G.part[i] = at<float>(ws[i], W.part);
        G.amax[i] = at<float>(ws[i], W.amax);
        G.ncols[i] = P.n_lead;
        ks = W.rp_ksplit;  // depends on T and d_in only: the same for every linear of the group
    }
    QE_TRY_HIP(launch_route_pass_group(reinterpret_cast<const uint16_t*>(x), T, lins[0]->d_in, G, n, ks, s));
    // The rest as one launch per step for the whole group when every linear is routed with the
    // same padded rank and token order rule; else linear by linear.
    bool grouped = true;
    const bool ko0 = keep_order ? keep_order[0] : false;
    for (int i = 0; i < n; ++i)
        grouped = grouped && lins[i]->n_routed > 0 && expert[i] && v[i] &&
                  prep_layout(lins[i]).rr_pad == prep_layout(lins[0]).rr_pad &&
                  (keep_order ? keep_order[i] : false) == ko0;
    if (!grouped) {
        for (int i = 0; i < n; ++i) {
            int st = run_prologue_rest(lins[i], x, T, codes[i], s_x[i], u[i], v[i], expert[i], perm[i], ws[i], s,
                                       keep_order ? keep_order[i] : false);
            if (st) return st;
        }
        return QE_OK;
    }
    FinishGroup F{};
    EqGroup E{};
    int ksq = 0;
    for (int i = 0; i < n; ++i) {
        const qe_linear* lin = lins[i];
        const PrepLayout P = prep_layout(lin);
        const WsLayout W = ws_layout(lin, T);
        const int qmax = (1 << (lin->a_bits - 1)) - 1;
        FinishLinear& f = F.lin[i];
        f.part = at<const float>(ws[i], W.part);
        f.amax = at<const float>(ws[i], W.amax);
        f.ncols = P.n_lead;
        f.r_s = lin->r_shared;
        f.rs_pad = P.rs_pad;
        f.router_col = P.col_router;
        f.n_r = lin->n_routed;
        f.qmax = qmax;
        f.expert = expert[i];
        f.u = u[i];
        f.s_x = s_x[i];
        EqLinear& e = E.lin[i];
        e.smooth = at<const float>(lin->prep, P.smooth);
        e.inv_smooth = at<const float>(lin->prep, P.inv_smooth);
        e.s_x = s_x[i];
        e.qmax = qmax;
        e.expert = expert[i];
        e.n_r = lin->n_routed;
        e.mt_re = at<const uint16_t>(lin->prep, P.mt) + (size_t)P.col_re * lin->d_in;
        e.r_r = lin->r_routed;
        e.perm = perm[i] ? perm[i] : at<int32_t>(ws[i], W.perm);
        e.vpart = at<float>(ws[i], W.vpart);
        e.codes = codes[i];
        e.v = v[i];
        ksq = W.eq_ksplit;  // depends on T and d_in only
    }
    QE_TRY_HIP(launch_route_finish_group(F, n, ks, T, s));
    QE_TRY_HIP(launch_expert_quant_group(reinterpret_cast<const uint16_t*>(x), T, lins[0]->d_in, E, n,
                                         prep_layout(lins[0]).rr_pad, ksq, ko0, s));
    return QE_OK;
}

// The main products of a group in one launch when every linear takes the 128-token-tile fast
// path (A6/A8, float32 y, ranks <= 32) and the combined grid fills the chip; false: nothing was
// launched and the caller runs the linears' products one by one.
static bool try_group_gemm(const qe_linear* const* lins, int n, int T, int8_t* const* codes, float* const* s_x,
                           uint16_t* const* u, uint16_t* const* v, int32_t* const* expert, int32_t* const* perm,
                           float* const* y, hipStream_t s, int* status) {
    *status = QE_OK;
    if (n < 1 || n > GG_MAX || T <= kSkinnyMaxT) return false;
    GemmGroup G{};
    G.n = n;
    G.T = T;
    for (int i = 0; i < n; ++i) {
        const qe_linear* lin = lins[i];
        if (lin->a_bits == 16 || lin->y_dtype != QE_F32) return false;
        const PrepLayout P = prep_layout(lin);
        const WsLayout W = ws_layout(lin, T);
        if (W.gemm_ksplit > 1 || P.rs_pad > 32 || P.rr_pad > 32) return false;
        GemmLinear& a = G.lin[i];
        a.codes = codes[i];
        a.s_x = s_x[i];
        a.w_tiled = at<const uint8_t>(lin->prep, P.w_tiled);
        a.w_scale = at<const float>(lin->prep, P.w_scale);
        a.u = (P.rs_pad > 0 && u[i]) ? u[i] : nullptr;
        a.bt_s = a.u ? at<const uint16_t>(lin->prep, P.bt_s) : nullptr;
        const bool routed = P.rr_pad > 0 && v[i] && expert[i];
        a.v = routed ? v[i] : nullptr;
        a.expert = routed ? expert[i] : nullptr;
        a.bt_r = routed ? at<const uint16_t>(lin->prep, P.bt_r) : nullptr;
        a.perm = perm[i];
        a.y = y[i];
        a.d_in = lin->d_in;
        a.d_out = lin->d_out;
        a.rs_pad = a.u ? P.rs_pad : 0;
        a.rr_pad = routed ? P.rr_pad : 0;
        a.n_r = routed ? lin->n_routed : 0;
    }
    const hipError_t e = launch_gemm_w4_group(G, s);
    if (e == hipErrorInvalidValue) return false;  // a grid not a multiple of 8: nothing launched
    *status = e == hipSuccess ? QE_OK : hip_fail(e);
    return true;
}

int qe_group_gemm(const qe_linear* const* lins, int32_t n_lin, const int8_t* const* codes, const float* const* s_x,
                  int32_t T, const uint16_t* const* u, const uint16_t* const* v, const int32_t* const* expert,
                  const int32_t* const* perm, float* const* y, void* const* ws, const size_t* ws_bytes, void* stream) {
    QE_CHECK(lins && n_lin >= 1 && n_lin <= RG_MAX && codes && s_x && u && v && expert && perm && y && ws && ws_bytes,
             QE_ERR_INVALID_ARG);
    for (int i = 0; i < n_lin; ++i) {
        QE_CHECK(lins[i] && lins[i]->a_bits != 16, QE_ERR_INVALID_ARG);
        int st = validate_forward_common(lins[i], T, QE_BF16, nullptr, ws[i], ws_bytes[i]);
        if (st) return st;
        if (T == 0) continue;
        QE_CHECK(codes[i] && s_x[i] && y[i], QE_ERR_INVALID_ARG);
        QE_CHECK(aligned16(codes[i]) && aligned16(y[i]), QE_ERR_ALIGNMENT);
        QE_CHECK((v[i] == nullptr) == (expert[i] == nullptr), QE_ERR_INVALID_ARG);
    }
    if (T == 0) return QE_OK;
    hipStream_t s = S(stream);
    int st = QE_OK;
    if (try_group_gemm(lins, n_lin, T, const_cast<int8_t* const*>(codes), const_cast<float* const*>(s_x),
                       const_cast<uint16_t* const*>(u), const_cast<uint16_t* const*>(v),
                       const_cast<int32_t* const*>(expert), const_cast<int32_t* const*>(perm), y, s, &st))
        return st;
    for (int i = 0; i < n_lin; ++i) {
        st = run_gemm(lins[i], codes[i], s_x[i], nullptr, QE_BF16, T, u[i], v[i], expert[i], perm[i], y[i], nullptr,
                      ws[i], s);
        if (st) return st;
    }
    return QE_OK;
}

int qe_group_prologue(const qe_linear* const* lins, int32_t n_lin, const void* x, int32_t x_dtype, int32_t T,
                      int8_t* const* codes, float* const* s_x, uint16_t* const* u, uint16_t* const* v,
                      int32_t* const* expert, int32_t* const* perm, void* const* ws, const size_t* ws_bytes,
                      void* stream) {
    int st = validate_group(lins, n_lin, T, x_dtype, x, ws, ws_bytes);
    if (st) return st;
    QE_CHECK(codes && s_x && u && v && expert && perm, QE_ERR_INVALID_ARG);
    if (T == 0) return QE_OK;
    QE_CHECK(x != nullptr, QE_ERR_INVALID_ARG);
    for (int i = 0; i < n_lin; ++i) {
        const qe_linear* lin = lins[i];
        QE_CHECK(lin->a_bits == 16 ? (codes[i] == nullptr && s_x[i] == nullptr) : (codes[i] && s_x[i]),
                 QE_ERR_INVALID_ARG);
        QE_CHECK((lin->r_shared > 0) == (u[i] != nullptr), QE_ERR_INVALID_ARG);
        QE_CHECK((lin->n_routed > 0) == (v[i] != nullptr) && (lin->n_routed > 0) == (expert[i] != nullptr),
                 QE_ERR_INVALID_ARG);
        QE_CHECK(!perm[i] || lin->n_routed > 0, QE_ERR_INVALID_ARG);
        if (codes[i]) QE_CHECK(aligned16(codes[i]), QE_ERR_ALIGNMENT);
    }
    return run_group_prologue(lins, n_lin, x, x_dtype, T, codes, s_x, u, v, expert, perm, ws, S(stream), nullptr);
}

int qe_group_forward(const qe_linear* const* lins, int32_t n_lin, const void* x, int32_t x_dtype, int32_t T,
                     float* const* y, int32_t* const* expert_out, void* const* ws, const size_t* ws_bytes,
                     void* stream) {
    int st = validate_group(lins, n_lin, T, x_dtype, x, ws, ws_bytes);
    if (st) return st;
    QE_CHECK(y, QE_ERR_INVALID_ARG);
    if (T == 0) return QE_OK;
    QE_CHECK(x != nullptr, QE_ERR_INVALID_ARG);
    for (int i = 0; i < n_lin; ++i) QE_CHECK(y[i] && aligned16(y[i]), y[i] ? QE_ERR_ALIGNMENT : QE_ERR_INVALID_ARG);
    if (!group_route_pass(lins, n_lin, x_dtype, T)) {  // the linears one by one
        for (int i = 0; i < n_lin; ++i) {
            st = qe_linear_forward(lins[i], x, x_dtype, T, y[i], expert_out ? expert_out[i] : nullptr, ws[i],
                                   ws_bytes[i], stream);
            if (st) return st;
        }
        return QE_OK;
    }
    hipStream_t s = S(stream);
    int8_t* codes[RG_MAX];
    float* s_x[RG_MAX];
    uint16_t *u[RG_MAX], *v[RG_MAX];
    int32_t *expert[RG_MAX], *perm[RG_MAX];
    bool keep[RG_MAX];
    for (int i = 0; i < n_lin; ++i) {  // the buffers qe_linear_forward takes from each workspace
        const qe_linear* lin = lins[i];
        const PrepLayout P = prep_layout(lin);
        const WsLayout W = ws_layout(lin, T);
        const bool route = lin->n_routed > 0;
        expert[i] = route ? (expert_out && expert_out[i] ? expert_out[i] : at<int32_t>(ws[i], W.expert)) : nullptr;
        u[i] = P.rs_pad > 0 ? at<uint16_t>(ws[i], W.u) : nullptr;
        v[i] = route ? at<uint16_t>(ws[i], W.v) : nullptr;
        codes[i] = at<int8_t>(ws[i], W.codes);
        s_x[i] = at<float>(ws[i], W.s_x);
        keep[i] = expert_quant_few(T) && W.gemm_ksplit > 1;
        perm[i] = (route && !keep[i]) ? at<int32_t>(ws[i], W.perm) : nullptr;
    }
    st = run_group_prologue(lins, n_lin, x, x_dtype, T, codes, s_x, u, v, expert, perm, ws, s, keep);
    if (st) return st;
    if (try_group_gemm(lins, n_lin, T, codes, s_x, u, v, expert, perm, y, s, &st)) return st;
    for (int i = 0; i < n_lin; ++i) {
        st = run_gemm(lins[i], codes[i], s_x[i], x, x_dtype, T, u[i], v[i], expert[i], perm[i], y[i], nullptr, ws[i], s);
        if (st) return st;
    }
    return QE_OK;
}

size_t qe_noalloc_scratch_bytes(void) { return qe::kNoAllocScratchBytes; }

int qe_linear_forward_noalloc(const qe_linear* lin, const void* x, int32_t x_dtype, int32_t T, float* y,
                              int32_t* expert_out, void* stream) {
    int st = validate_linear(lin);
    if (st) return st;
    QE_CHECK(T >= 0, QE_ERR_INVALID_ARG);
    if (T == 0) return QE_OK;
    QE_CHECK(ws_layout(lin, T).total <= qe::kNoAllocScratchBytes, QE_ERR_WORKSPACE);
    void* scratch_dev = nullptr;
    st = qe::noalloc_scratch(&scratch_dev);
    if (st) return st;
    return qe_linear_forward(lin, x, x_dtype, T, y, expert_out, scratch_dev, qe::kNoAllocScratchBytes, stream);
}

// ------------------------------------------------------------------ a8
int qe_colmean_abs(const void* W, int32_t dtype, int32_t d_out, int32_t d_in, float* w, void* stream) {
    QE_CHECK(W && w, QE_ERR_INVALID_ARG);
    QE_CHECK(d_out > 0 && d_in > 0, QE_ERR_INVALID_ARG);
    QE_CHECK(dtype == QE_F32 || dtype == QE_BF16, QE_ERR_INVALID_ARG);
    QE_CHECK(aligned16(W) && aligned16(w), QE_ERR_ALIGNMENT);
    QE_TRY_HIP(launch_colmean(W, dtype, d_out, d_in, w, S(stream)));
    return QE_OK;
}

int qe_channel_topk(const void* x, int32_t x_dtype, const float* w, int32_t T, int32_t d_in, int32_t k, int32_t* topk,
                    uint32_t* hist, void* stream) {
    QE_CHECK(T >= 0 && d_in > 0, QE_ERR_INVALID_ARG);
    QE_CHECK(x_dtype == QE_F32 || x_dtype == QE_BF16, QE_ERR_INVALID_ARG);
    QE_CHECK(k >= 1 && k <= d_in, QE_ERR_INVALID_ARG);
    QE_CHECK(k <= 1024 && d_in <= 32768, QE_ERR_UNSUPPORTED);
    if (T == 0) return QE_OK;
    QE_CHECK(x && w && hist, QE_ERR_INVALID_ARG);
    QE_CHECK(aligned16(x) && aligned16(w) && aligned16(hist), QE_ERR_ALIGNMENT);
    if (topk) QE_CHECK(aligned16(topk), QE_ERR_ALIGNMENT);
    QE_TRY_HIP(launch_topk(x, x_dtype, w, T, d_in, k, topk, hist, S(stream)));
    return QE_OK;
}

// ------------------------------------------------------ channel partition and clustering
int qe_partition_channels(const uint32_t* hist, int32_t d_in, int32_t k, int32_t n_r, int32_t* indep,
                          int32_t* dep, int32_t* slot) {
    QE_CHECK(hist && indep && dep, QE_ERR_INVALID_ARG);
    QE_CHECK(d_in >= 1 && k >= 1 && n_r >= 1, QE_ERR_INVALID_ARG);
    QE_CHECK((int64_t)k * (1 + (int64_t)n_r) <= d_in, QE_ERR_INVALID_ARG);
    std::vector<int32_t> order(d_in);
    frequency_order(hist, d_in, order.data());
    const int n_dep = k * n_r;
    std::copy(order.begin(), order.begin() + k, indep);
    std::copy(order.begin() + k, order.begin() + k + n_dep, dep);
    if (slot) {
        std::fill(slot, slot + d_in, -1);
        for (int m = 0; m < n_dep; ++m) slot[dep[m]] = m;
    }
    return QE_OK;
}

size_t qe_cooccur_workspace_bytes(int32_t T, int32_t n_dep) {
    if (T < 0 || n_dep < 1 || n_dep > 8192) return 0;
    return cooccur_workspace_bytes(T, n_dep);
}

int qe_cooccur(const int32_t* topk, int32_t T, int32_t k, const int32_t* slot, int32_t d_in, int32_t n_dep,
               uint32_t* cooc, void* ws, size_t ws_bytes, void* stream) {
    QE_CHECK(T >= 0 && d_in >= 1 && n_dep >= 1 && k >= 1 && k <= d_in, QE_ERR_INVALID_ARG);
    QE_CHECK(k <= 1024 && n_dep <= 8192, QE_ERR_UNSUPPORTED);
    if (T == 0) return QE_OK;
    QE_CHECK(topk && slot && cooc, QE_ERR_INVALID_ARG);
    QE_CHECK(aligned16(topk) && aligned16(slot) && aligned16(cooc), QE_ERR_ALIGNMENT);
    QE_CHECK(ws != nullptr && ws_bytes >= cooccur_workspace_bytes(T, n_dep), QE_ERR_WORKSPACE);
    QE_CHECK(aligned16(ws), QE_ERR_ALIGNMENT);
    QE_TRY_HIP(launch_cooccur(topk, T, k, slot, d_in, n_dep, cooc, ws, S(stream)));
    return QE_OK;
}

int qe_cluster_channels(const uint32_t* cooc, int32_t n_dep, int64_t T, int32_t n_clusters, double threshold,
                        int32_t* labels, double* similarity, double* eigvals, double* embedding) {
    QE_CHECK(cooc && labels, QE_ERR_INVALID_ARG);
    QE_CHECK(n_dep >= 1 && T >= 1 && n_clusters >= 1 && n_clusters <= n_dep, QE_ERR_INVALID_ARG);
    QE_CHECK(threshold >= 0.0 && threshold <= 1.0, QE_ERR_INVALID_ARG);  // also rejects NaN
    QE_CHECK(n_dep <= 2048, QE_ERR_UNSUPPORTED);
    const size_t n = (size_t)n_dep;
    for (size_t i = 0; i < n; ++i) {
        const uint32_t cii = cooc[i * n + i];
        QE_CHECK((int64_t)cii <= T, QE_ERR_INVALID_ARG);
        for (size_t j = 0; j < n; ++j) {
            const uint32_t cij = cooc[i * n + j];
            QE_CHECK(cij == cooc[j * n + i] && cij <= cii && cij <= cooc[j * n + j], QE_ERR_INVALID_ARG);
        }
    }
    if (spectral_cluster(cooc, n_dep, T, n_clusters, threshold, labels, similarity, eigvals, embedding) != 0)
        return QE_ERR_UNSUPPORTED;
    return QE_OK;
}

// ------------------------------------------------------------------ top-2 routing
// qe_linear_forward with the two routed experts of smallest score per token: the forward (its
// fused first expert), then the router scores, the best other expert, its adapter input and its
// term through the grouped routed path (added into y).
size_t qe_top2_workspace_bytes(const qe_linear* lin, int32_t T) {
    const size_t base = qe_workspace_bytes(lin, T);
    if (base == 0 || lin->n_routed < 2 || T < 0) return 0;
    const size_t t4 = align256((size_t)std::max(T, 1) * 4);
    const PrepLayout P = prep_layout(lin);
    return align256(base) + 4 * t4 + align256((size_t)std::max(T, 1) * lin->n_routed * 4) +
           2 * align256(((size_t)lin->n_routed + 1) * 4) + align256((size_t)std::max(T, 1) * P.rr_pad * 2);
}

int qe_linear_forward_top2(const qe_linear* lin, const void* x, int32_t x_dtype, int32_t T, float* y,
                           int32_t* expert_out, int32_t* expert2_out, void* ws, size_t ws_bytes, void* stream) {
    const size_t need = qe_top2_workspace_bytes(lin, T);
    QE_CHECK(lin && lin->n_routed >= 2 && need > 0, QE_ERR_INVALID_ARG);
    QE_CHECK(T <= 65535, QE_ERR_UNSUPPORTED);
    QE_CHECK(lin->y_dtype == QE_F32, QE_ERR_UNSUPPORTED);  // the second expert is added into y
    QE_CHECK(ws_bytes >= need, QE_ERR_WORKSPACE);
    const size_t base = qe_workspace_bytes(lin, T);
    if (T == 0) return validate_forward_common(lin, T, x_dtype, x, ws, ws_bytes);
    char* p = static_cast<char*>(ws) + align256(base);
    const size_t t4 = align256((size_t)T * 4);
    int32_t* e1 = reinterpret_cast<int32_t*>(p);
    int32_t* e2 = reinterpret_cast<int32_t*>(p + t4);
    int32_t* perm = reinterpret_cast<int32_t*>(p + 2 * t4);
    int32_t* e_tmp = reinterpret_cast<int32_t*>(p + 3 * t4);
    float* scores = reinterpret_cast<float*>(p + 4 * t4);
    char* q = p + 4 * t4 + align256((size_t)T * lin->n_routed * 4);
    int32_t* offsets = reinterpret_cast<int32_t*>(q);
    int32_t* counts = reinterpret_cast<int32_t*>(q + align256(((size_t)lin->n_routed + 1) * 4));
    uint16_t* v2 = reinterpret_cast<uint16_t*>(q + 2 * align256(((size_t)lin->n_routed + 1) * 4));
    const PrepLayout P = prep_layout(lin);
    const WsLayout W = ws_layout(lin, T);
    hipStream_t s = S(stream);
    if (lin->a_bits != 16 && lin->w_bits == 4 && T > kSkinnyMaxT &&
        gemm_w4_top2_ok(T, lin->d_out, P.rs_pad, P.rr_pad, W.gemm_ksplit, lin->y_dtype == QE_BF16)) {
        // Both routed corrections in the main product's epilogue: the prologue also gives each
        // token's second expert (from the same router scores), one more pass of x onto the routed
        // experts' input columns gives its v2, and every output is stored once.
        int st = validate_forward_common(lin, T, x_dtype, x, ws, ws_bytes);
        if (st) return st;
        QE_CHECK(x && y, QE_ERR_INVALID_ARG);
        QE_CHECK(aligned16(y), QE_ERR_ALIGNMENT);
        int8_t* codes = at<int8_t>(ws, W.codes);
        float* s_x = at<float>(ws, W.s_x);
        uint16_t* u = P.rs_pad > 0 ? at<uint16_t>(ws, W.u) : nullptr;
        uint16_t* v = at<uint16_t>(ws, W.v);
        int32_t* perm_g = at<int32_t>(ws, W.perm);
        st = run_prologue(lin, x, x_dtype, T, codes, s_x, u, v, e1, perm_g, ws, s, false, e2);
        if (st) return st;
        const int nc = lin->n_routed * P.rr_pad, nc_pad = (nc + 15) / 16 * 16;
        float* part = at<float>(ws, W.part);
        int ks = 0;
        st = xpass_partials(lin, x, x_dtype, T, P.col_re, nc, nc_pad, part, ws, s, &ks);
        if (st) return st;
        QE_TRY_HIP(launch_xproj_finish(part, ks, T, nc_pad, P.col_re, -1, lin->r_shared, P.rs_pad, P.col_re,
                                       lin->n_routed, lin->r_routed, P.rr_pad, -1, e2, nullptr, nullptr, nullptr, v2,
                                       s));
        QE_TRY_HIP(launch_gemm_w4_top2(codes, s_x, at<const uint8_t>(lin->prep, P.w_tiled),
                                       at<const float>(lin->prep, P.w_scale), T, lin->d_in, lin->d_out, u,
                                       P.rs_pad > 0 ? at<const uint16_t>(lin->prep, P.bt_s) : nullptr, P.rs_pad, v, e1,
                                       v2, e2, at<const uint16_t>(lin->prep, P.bt_r), P.rr_pad, lin->n_routed, perm_g,
                                       y, s));
        if (expert_out) QE_TRY_HIP(hipMemcpyAsync(expert_out, e1, (size_t)T * 4, hipMemcpyDeviceToDevice, s));
        if (expert2_out) QE_TRY_HIP(hipMemcpyAsync(expert2_out, e2, (size_t)T * 4, hipMemcpyDeviceToDevice, s));
        return QE_OK;
    }
    int st = qe_linear_forward(lin, x, x_dtype, T, y, e1, ws, base, stream);
    if (st) return st;
    // one pass of x onto the router and every routed expert's input columns; the finish runs twice
    // on its partials: the scores first, then v of the second expert
    const int c0 = std::min(P.col_re, P.col_router);
    const int c1 = std::max(P.col_re + lin->n_routed * P.rr_pad, P.col_router + lin->n_routed);
    const int nc = c1 - c0, nc_pad = (nc + 15) / 16 * 16;
    float* part = at<float>(ws, W.part);
    int ks = 0;
    st = xpass_partials(lin, x, x_dtype, T, c0, nc, nc_pad, part, ws, s, &ks);
    if (st) return st;
    QE_TRY_HIP(launch_xproj_finish(part, ks, T, nc_pad, c0, -1, lin->r_shared, P.rs_pad, -1, lin->n_routed,
                                   lin->r_routed, P.rr_pad, P.col_router, nullptr, scores, e_tmp, nullptr, nullptr, s));
    QE_TRY_HIP(launch_second_expert(scores, e1, T, lin->n_routed, e2, s));
    uint16_t* v = at<uint16_t>(ws, W.v);
    QE_TRY_HIP(launch_xproj_finish(part, ks, T, nc_pad, c0, -1, lin->r_shared, P.rs_pad, P.col_re, lin->n_routed,
                                   lin->r_routed, P.rr_pad, -1, e2, nullptr, nullptr, nullptr, v, s));
    QE_TRY_HIP(launch_bucket(e2, T, lin->n_routed, counts, offsets, perm, s));
    QE_TRY_HIP(launch_routed_lora(v, P.rr_pad, offsets, perm, lin->n_routed, at<const uint16_t>(lin->prep, P.bt_r), T,
                                  lin->d_out, y, s));
    if (expert_out) QE_TRY_HIP(hipMemcpyAsync(expert_out, e1, (size_t)T * 4, hipMemcpyDeviceToDevice, s));
    if (expert2_out) QE_TRY_HIP(hipMemcpyAsync(expert2_out, e2, (size_t)T * 4, hipMemcpyDeviceToDevice, s));
    return QE_OK;
}

// ------------------------------------------------------------------ expert construction
namespace {
int lowrank_status(hipError_t e) {
    if (e == hipSuccess) return QE_OK;
    if (e == hipErrorNotSupported) return QE_ERR_UNSUPPORTED;  // eigenvalue iteration did not converge
    return hip_fail(e);
}
}  // namespace

int qe_quant_error(const float* W_f, const float* s, int32_t d_out, int32_t d_in, int32_t w_bits, float* E,
                   void* stream) {
    QE_CHECK(W_f && E && d_out > 0 && d_in > 0 && (w_bits == 3 || w_bits == 4), QE_ERR_INVALID_ARG);
    QE_CHECK(aligned16(W_f) && aligned16(E) && (!s || aligned16(s)), QE_ERR_ALIGNMENT);
    QE_TRY_HIP(launch_quant_error(W_f, s, d_out, d_in, w_bits, E, S(stream)));
    return QE_OK;
}

size_t qe_channel_rms_workspace_bytes(int32_t T, int32_t d_in) {
    return T > 0 && d_in > 0 ? channel_rms_workspace_bytes(T, d_in) : 0;
}

int qe_channel_rms(const void* x, int32_t x_dtype, int32_t T, int32_t d_in, float* c, void* ws, size_t ws_bytes,
                   void* stream) {
    QE_CHECK(x && c && ws && T > 0 && d_in > 0 && (x_dtype == QE_F32 || x_dtype == QE_BF16), QE_ERR_INVALID_ARG);
    QE_CHECK(aligned16(x) && aligned16(c) && aligned16(ws), QE_ERR_ALIGNMENT);
    QE_CHECK(ws_bytes >= channel_rms_workspace_bytes(T, d_in), QE_ERR_WORKSPACE);
    QE_TRY_HIP(launch_channel_rms(x, x_dtype, T, d_in, c, ws, S(stream)));
    return QE_OK;
}

int qe_sub_lowrank(float* E, int32_t d_out, int32_t d_in, const float* A, const float* B, int32_t r, void* stream) {
    QE_CHECK(E && A && B && d_out > 0 && d_in > 0 && r >= 1 && r <= 64, QE_ERR_INVALID_ARG);
    QE_CHECK(aligned16(E) && aligned16(A) && aligned16(B), QE_ERR_ALIGNMENT);
    QE_TRY_HIP(launch_sub_lowrank(E, d_out, d_in, A, B, r, S(stream)));
    return QE_OK;
}

size_t qe_lowrank_workspace_bytes(int32_t d_out, int32_t d_in, int32_t k) {
    return d_out > 0 && d_in > 0 && k > 0 ? lowrank_workspace_bytes(d_out, d_in, k) : 0;
}

int qe_lowrank_fit(const float* E, int32_t d_out, int32_t d_in, const float* w, const float* omega, int32_t k,
                   int32_t rank, int32_t power_iters, float* A, float* B, double* sigma, void* ws, size_t ws_bytes,
                   void* stream) {
    QE_CHECK(E && omega && A && B && sigma && ws, QE_ERR_INVALID_ARG);
    QE_CHECK(d_out > 0 && d_in > 0 && k >= 1 && k <= 128 && k <= d_in && k <= d_out, QE_ERR_INVALID_ARG);
    QE_CHECK(rank >= 1 && rank <= k && power_iters >= 0 && power_iters <= 16, QE_ERR_INVALID_ARG);
    QE_CHECK(aligned16(E) && aligned16(omega) && aligned16(ws) && (!w || aligned16(w)), QE_ERR_ALIGNMENT);
    QE_CHECK(ws_bytes >= lowrank_workspace_bytes(d_out, d_in, k), QE_ERR_WORKSPACE);
    return lowrank_status(lowrank_fit(E, d_out, d_in, w, omega, k, rank, power_iters, A, B, sigma, ws, S(stream)));
}

size_t qe_build_experts_workspace_bytes(int32_t d_out, int32_t d_in, int32_t k, int32_t r_max) {
    return d_out > 0 && d_in > 0 && k > 0 && r_max >= 0 ? build_experts_workspace_bytes(d_out, d_in, k, r_max) : 0;
}

int qe_build_experts(const float* W_f, const float* s, int32_t d_out, int32_t d_in, int32_t w_bits, const float* c,
                     const int32_t* dep_channels, const int32_t* labels, int32_t n_dep, int32_t n_routed,
                     int32_t r_shared, int32_t r_routed, const float* omegas, int32_t k, int32_t power_iters,
                     float* A_s, float* B_s, float* A_r, float* B_r, double* sigma_s, double* sigma_r, void* ws,
                     size_t ws_bytes, void* stream) {
    QE_CHECK(W_f && c && omegas && ws && (w_bits == 3 || w_bits == 4), QE_ERR_INVALID_ARG);
    QE_CHECK(d_out > 0 && d_in > 0 && k >= 1 && k <= 128 && k <= d_in && k <= d_out, QE_ERR_INVALID_ARG);
    QE_CHECK(r_shared >= 0 && r_shared <= 64 && r_shared <= k && power_iters >= 0 && power_iters <= 16,
             QE_ERR_INVALID_ARG);
    QE_CHECK(n_routed >= 0 && n_routed <= 16, QE_ERR_INVALID_ARG);
    if (r_shared > 0) QE_CHECK(A_s && B_s && sigma_s, QE_ERR_INVALID_ARG);
    if (n_routed > 0) {
        QE_CHECK(r_routed >= 1 && r_routed <= 64 && r_routed <= k, QE_ERR_INVALID_ARG);
        QE_CHECK(A_r && B_r && sigma_r && n_dep >= 0 && (n_dep == 0 || (dep_channels && labels)), QE_ERR_INVALID_ARG);
        for (int t = 0; t < n_dep; ++t)
            QE_CHECK(dep_channels[t] >= 0 && dep_channels[t] < d_in && labels[t] >= 0 && labels[t] < n_routed,
                     QE_ERR_INVALID_ARG);
    }
    QE_CHECK(aligned16(W_f) && aligned16(c) && aligned16(omegas) && aligned16(ws) && (!s || aligned16(s)),
             QE_ERR_ALIGNMENT);
    const int r_max = std::max(r_shared, n_routed > 0 ? r_routed : 0);
    QE_CHECK(ws_bytes >= build_experts_workspace_bytes(d_out, d_in, k, r_max), QE_ERR_WORKSPACE);
    return lowrank_status(build_experts(W_f, s, d_out, d_in, w_bits, c, dep_channels, labels, n_dep, n_routed,
                                        r_shared, n_routed > 0 ? r_routed : 0, omegas, k, power_iters, A_s, B_s, A_r,
                                        B_r, sigma_s, sigma_r, ws, S(stream)));
}

size_t qe_lowrank_cov_workspace_bytes(int32_t d_out, int32_t d_in, int32_t T, int32_t k) {
    return d_out > 0 && d_in > 0 && T > 0 && k > 0 ? lowrank_cov_workspace_bytes(d_out, d_in, T, k) : 0;
}

int qe_lowrank_fit_cov(const float* E, int32_t d_out, int32_t d_in, const float* X, int32_t T, const float* mask,
                       const float* omega, int32_t k, int32_t rank, int32_t power_iters, float* A, float* B,
                       double* sigma, void* ws, size_t ws_bytes, void* stream) {
    QE_CHECK(E && X && omega && A && B && sigma && ws, QE_ERR_INVALID_ARG);
    QE_CHECK(d_out > 0 && d_in > 0 && T > 0 && k >= 1 && k <= 128 && k <= d_out && k <= T, QE_ERR_INVALID_ARG);
    QE_CHECK(rank >= 1 && rank <= k && power_iters >= 0 && power_iters <= 16, QE_ERR_INVALID_ARG);
    QE_CHECK(aligned16(E) && aligned16(X) && aligned16(omega) && aligned16(ws) && (!mask || aligned16(mask)),
             QE_ERR_ALIGNMENT);
    QE_CHECK(ws_bytes >= lowrank_cov_workspace_bytes(d_out, d_in, T, k), QE_ERR_WORKSPACE);
    return lowrank_status(
        lowrank_fit_cov(E, d_out, d_in, X, T, mask, omega, k, rank, power_iters, A, B, sigma, ws, S(stream)));
}

size_t qe_build_experts_cov_workspace_bytes(int32_t d_out, int32_t d_in, int32_t T, int32_t k, int32_t r_max) {
    return d_out > 0 && d_in > 0 && T > 0 && k > 0 && r_max >= 0
               ? build_experts_cov_workspace_bytes(d_out, d_in, T, k, r_max)
               : 0;
}

int qe_build_experts_cov(const float* W_f, const float* s, int32_t d_out, int32_t d_in, int32_t w_bits,
                         const void* x, int32_t x_dtype, int32_t T, const int32_t* dep_channels,
                         const int32_t* labels, int32_t n_dep, int32_t n_routed, int32_t r_shared, int32_t r_routed,
                         const float* omegas, int32_t k, int32_t power_iters, float* A_s, float* B_s, float* A_r,
                         float* B_r, double* sigma_s, double* sigma_r, void* ws, size_t ws_bytes, void* stream) {
    QE_CHECK(W_f && x && omegas && ws && (w_bits == 3 || w_bits == 4), QE_ERR_INVALID_ARG);
    QE_CHECK(x_dtype == QE_F32 || x_dtype == QE_BF16, QE_ERR_INVALID_ARG);
    QE_CHECK(d_out > 0 && d_in > 0 && T > 0 && k >= 1 && k <= 128 && k <= d_out && k <= T, QE_ERR_INVALID_ARG);
    QE_CHECK(r_shared >= 0 && r_shared <= 64 && r_shared <= k && power_iters >= 0 && power_iters <= 16,
             QE_ERR_INVALID_ARG);
    QE_CHECK(n_routed >= 0 && n_routed <= 16, QE_ERR_INVALID_ARG);
    if (r_shared > 0) QE_CHECK(A_s && B_s && sigma_s, QE_ERR_INVALID_ARG);
    if (n_routed > 0) {
        QE_CHECK(r_routed >= 1 && r_routed <= 64 && r_routed <= k, QE_ERR_INVALID_ARG);
        QE_CHECK(A_r && B_r && sigma_r && n_dep >= 0 && (n_dep == 0 || (dep_channels && labels)), QE_ERR_INVALID_ARG);
        for (int t = 0; t < n_dep; ++t)
            QE_CHECK(dep_channels[t] >= 0 && dep_channels[t] < d_in && labels[t] >= 0 && labels[t] < n_routed,
                     QE_ERR_INVALID_ARG);
    }
    QE_CHECK(aligned16(W_f) && aligned16(x) && aligned16(omegas) && aligned16(ws) && (!s || aligned16(s)),
             QE_ERR_ALIGNMENT);
    const int r_max = std::max(r_shared, n_routed > 0 ? r_routed : 0);
    QE_CHECK(ws_bytes >= build_experts_cov_workspace_bytes(d_out, d_in, T, k, r_max), QE_ERR_WORKSPACE);
    return lowrank_status(build_experts_cov(W_f, s, d_out, d_in, w_bits, x, x_dtype, T, dep_channels, labels, n_dep,
                                            n_routed, r_shared, n_routed > 0 ? r_routed : 0, omegas, k, power_iters,
                                            A_s, B_s, A_r, B_r, sigma_s, sigma_r, ws, S(stream)));
}

size_t qe_router_targets_workspace_bytes(int32_t d_out, int32_t d_in, int32_t n_routed, int32_t r_routed) {
    return d_out > 0 && d_in > 0 && n_routed > 0 && r_routed > 0
               ? router_targets_workspace_bytes(d_out, d_in, n_routed, r_routed)
               : 0;
}

int qe_router_targets(const float* E1, int32_t d_out, int32_t d_in, const void* x, int32_t x_dtype, int32_t T,
                      const float* A_r, const float* B_r, int32_t n_routed, int32_t r_routed, float* target, void* ws,
                      size_t ws_bytes, void* stream) {
    QE_CHECK(E1 && x && A_r && B_r && target && ws && d_out > 0 && d_in > 0 && T > 0, QE_ERR_INVALID_ARG);
    QE_CHECK(n_routed >= 1 && n_routed <= 16 && r_routed >= 1 && r_routed <= 64, QE_ERR_INVALID_ARG);
    QE_CHECK(x_dtype == QE_F32 || x_dtype == QE_BF16, QE_ERR_INVALID_ARG);
    for (const void* q : {(const void*)E1, x, (const void*)A_r, (const void*)B_r, (const void*)target, (const void*)ws})
        QE_CHECK(aligned16(q), QE_ERR_ALIGNMENT);
    QE_CHECK(ws_bytes >= router_targets_workspace_bytes(d_out, d_in, n_routed, r_routed), QE_ERR_WORKSPACE);
    QE_TRY_HIP(router_targets(E1, d_out, d_in, x, x_dtype, T, A_r, B_r, n_routed, r_routed, target, ws, S(stream)));
    return QE_OK;
}

size_t qe_router_fit_workspace_bytes(int32_t T, int32_t d_in, int32_t n_routed) {
    return T > 0 && d_in > 0 && n_routed > 0 ? router_fit_workspace_bytes(T, d_in, n_routed) : 0;
}

int qe_router_fit(const void* x, int32_t x_dtype, int32_t T, int32_t d_in, const float* target, int32_t n_routed,
                  double ridge, int32_t max_iters, double tol, float* R, int32_t* iters_done, void* ws, size_t ws_bytes,
                  void* stream) {
    QE_CHECK(x && target && R && ws && T > 0 && d_in > 0 && n_routed >= 1 && n_routed <= 16, QE_ERR_INVALID_ARG);
    QE_CHECK(x_dtype == QE_F32 || x_dtype == QE_BF16, QE_ERR_INVALID_ARG);
    QE_CHECK(ridge >= 0.0 && max_iters >= 0 && max_iters <= 100000 && tol >= 0.0, QE_ERR_INVALID_ARG);
    QE_CHECK(aligned16(x) && aligned16(target) && aligned16(ws), QE_ERR_ALIGNMENT);
    QE_CHECK(ws_bytes >= router_fit_workspace_bytes(T, d_in, n_routed), QE_ERR_WORKSPACE);
    int done = 0;
    QE_TRY_HIP(router_fit(x, x_dtype, T, d_in, target, n_routed, ridge, max_iters, tol, R, &done, ws, S(stream)));
    if (iters_done) *iters_done = done;
    return QE_OK;
}

// ------------------------------------------------------------------ measurement aids
int qe_probe_mfma_i8(int32_t* out, int32_t blocks, int32_t iters, int32_t operands, double* ops, void* stream) {
    QE_CHECK(out && blocks >= 1 && iters >= 1 && (operands == 0 || operands == 1), QE_ERR_INVALID_ARG);
    QE_CHECK(aligned16(out), QE_ERR_ALIGNMENT);
    QE_TRY_HIP(launch_probe_mfma_i8(out, blocks, iters, operands, S(stream)));
    if (ops) *ops = probe_mfma_i8_ops(blocks, iters);
    return QE_OK;
}

int qe_probe_mfma_bf16(float* out, int32_t blocks, int32_t iters, int32_t operands, double* flops, void* stream) {
    QE_CHECK(out && blocks >= 1 && iters >= 1 && (operands == 0 || operands == 1), QE_ERR_INVALID_ARG);
    QE_CHECK(aligned16(out), QE_ERR_ALIGNMENT);
    QE_TRY_HIP(launch_probe_mfma_bf16(out, blocks, iters, operands, S(stream)));
    if (flops) *flops = probe_mfma_bf16_flops(blocks, iters);
    return QE_OK;
}

int qe_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
    QE_CHECK(src && dst && bytes % 16 == 0, QE_ERR_INVALID_ARG);
    QE_CHECK(aligned16(src) && aligned16(dst), QE_ERR_ALIGNMENT);
    const char *a = static_cast<const char*>(src), *b = static_cast<const char*>(dst);
    QE_CHECK(a + bytes <= b || b + bytes <= a, QE_ERR_INVALID_ARG);
    if (bytes == 0) return QE_OK;
    QE_TRY_HIP(launch_probe_copy(src, dst, bytes, S(stream)));
    return QE_OK;
}

size_t qe_probe_read_sink_bytes(void) { return probe_read_sink_words() * sizeof(uint32_t); }

int qe_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    QE_CHECK(src && sink && bytes % 16 == 0, QE_ERR_INVALID_ARG);
    QE_CHECK(aligned16(src) && aligned16(sink), QE_ERR_ALIGNMENT);
    if (bytes == 0) return QE_OK;
    QE_TRY_HIP(launch_probe_read(src, bytes, sink, S(stream)));
    return QE_OK;
}

// ------------------------------------------------------------------ cost
int qe_linear_cost(const qe_linear* lin, int32_t T, int32_t n_distinct, int32_t xb, double* int_macs,
                   double* adapter_macs, double* alg_bytes) {
    QE_CHECK(lin && T >= 0 && n_distinct >= 0 && (xb == 2 || xb == 4), QE_ERR_INVALID_ARG);
    QE_CHECK(lin->d_in > 0 && lin->d_out > 0, QE_ERR_INVALID_ARG);
    const double t = T, di = lin->d_in, dout = lin->d_out;
    const double rs = lin->r_shared, nr = lin->n_routed, rr = lin->n_routed > 0 ? lin->r_routed : 0;
    if (int_macs) *int_macs = t * di * dout;
    if (adapter_macs) *adapter_macs = t * (di + dout) * (rs + rr) + t * di * nr;
    if (alg_bytes) {
        double b = t * di * xb;                              // x read once
        b += di * dout * lin->w_bits / 8.0 + dout * 4.0;     // packed weights + scales
        if (lin->a_bits != 16) b += di * 4.0;                // smoothing vector
        b += t * dout * (lin->y_dtype == QE_BF16 ? 2.0 : 4.0);  // y written once
        b += (di + dout) * rs * 2.0;                         // shared expert
        b += std::min<double>(n_distinct, nr) * (di + dout) * rr * 2.0;  // selected routed experts
        b += di * nr * 2.0;                                  // router
        *alg_bytes = b;
    }
    return QE_OK;
}

}  // extern "C"
