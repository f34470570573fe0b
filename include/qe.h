/*
 * libqe -- the inference hot path of a Quant Experts (QE) linear layer on AMD
 * Instinct MI355X (gfx950), as a C ABI.
 *
 * What a QE linear computes (sources cited by page title and section):
 *   y = Q(x / s) . Q(W_f diag(s))^T            quantized main product
 *     + (x . A_s) . B_s                         shared expert (every token)
 *     + (x . A_e) . B_e,  e = argmin_j (x . R)_j  one routed expert per token
 *   - MCISLAB DeepRead summary "Quant Experts: Token-aware Adaptive Error
 *     Reconstruction with Mixture of Experts for Large Vision-Language Models
 *     Quantization", section "Method": shared low-rank expert for the global error,
 *     routed low-rank experts for token-specific error, a lightweight router that
 *     predicts each expert's remaining error and picks the smallest, channel-wise
 *     scaling before activation quantization, and the per-token statistic
 *     Top-k(|x_t| * Mean_row(|W_f|)).
 *   - thelatestinai.com listing of arXiv 2602.24059, Table 7: a QE linear costs
 *     s*d^2 + s*d*(2r + N_r) multiply-adds (dense adapters, one routed expert per
 *     token, one d x N_r router map); bit settings W4A6 / W4A8 / W3A16 (Tables 1-3).
 *
 * Conventions shared by every entry point
 *   - Return value: a qe_status (0 = QE_OK).  Arguments are validated on the host
 *     before anything is enqueued; on failure nothing is launched.  A failed HIP
 *     launch returns QE_ERR_HIP and its hipError_t is kept in qe_last_hip_error()
 *     (thread-local).  Faults inside kernels surface at the caller's next
 *     synchronisation.  No C++ exception crosses this ABI.  T == 0 is a no-op.
 *   - Memory: every pointer marked "device" is device memory allocated and owned
 *     by the caller; the library never allocates or frees memory and keeps no
 *     pointer after returning.  Buffers must stay valid until the work enqueued
 *     on `stream` has finished.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 *     stream).  Device entry points only enqueue work; none synchronises.
 *   - Layouts are row-major and dense.  bf16 tensors are passed as uint16_t bit
 *     patterns.  Device pointers must be 16-byte aligned (QE_ERR_ALIGNMENT).
 *   - Inputs must be finite; results for non-finite inputs are undefined.
 *   - The library holds no global mutable state except the thread-local error;
 *     calls on different streams may run concurrently as long as they do not
 *     share output or workspace buffers.
 */
#ifndef QE_H
#define QE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QE_OK = 0,
    QE_ERR_INVALID_ARG = 1,  /* bad shape, bit width, NULL required pointer, k > d_in ... */
    QE_ERR_UNSUPPORTED = 2,  /* valid but not implemented (e.g. W3 with A6/A8, d_in % 128 != 0) */
    QE_ERR_ALIGNMENT = 3,    /* a device pointer is not 16-byte aligned */
    QE_ERR_WORKSPACE = 4,    /* workspace / prepared buffer smaller than required */
    QE_ERR_HIP = 5           /* a HIP call failed; see qe_last_hip_error() */
} qe_status;

typedef enum { QE_F32 = 0, QE_BF16 = 1 } qe_dtype;

/* Shape and bit widths of one QE linear, plus its prepared parameter buffer.
 *   d_in, d_out  input / output channels (d_in > 0, d_out > 0)
 *   w_bits       4 (int4, per-output-channel symmetric) or 3 (3-bit, weight-only)
 *   a_bits       6 or 8 (per-token symmetric activation codes) with w_bits 4;
 *                16 (bf16 activations, no activation quantization) with w_bits 3 or 4
 *   r_shared     shared-expert rank, 0..64 (0 = no shared expert)
 *   n_routed     number of routed experts N_r, 0..16 (0 = no router, no routed expert)
 *   r_routed     routed-expert rank, 1..64 when n_routed > 0, else 0
 *   y_dtype      element type of the outputs y this linear writes: QE_F32 (0), or QE_BF16 (1),
 *                the round-to-nearest-even of the float32 value the QE_F32 setting writes
 *                (the bf16-output option of the decode settings, listing Tables 1-3 and 8);
 *                every `float* y` argument of the calls below then points at bf16 elements.
 *                qe_routed_lora and qe_linear_forward_top2 add into y and take QE_F32 only.
 *   prep         device buffer written by qe_prepare() (qe_prepared_bytes() bytes)
 * Kernel-path constraints: d_out % 16 == 0 and d_in % 128 == 0, and d_in <= 32768 when
 * a_bits is 6 or 8 (else QE_ERR_UNSUPPORTED).
 */
typedef struct qe_linear {
    int32_t d_in;
    int32_t d_out;
    int32_t w_bits;
    int32_t a_bits;
    int32_t r_shared;
    int32_t n_routed;
    int32_t r_routed;
    int32_t y_dtype;
    const void* prep;
} qe_linear;

/* Human-readable name of a status code (static storage). */
const char* qe_status_string(int status);

/* hipError_t of the last QE_ERR_HIP returned on this thread (0 if none). */
int qe_last_hip_error(void);

/* Library version string (static storage). */
const char* qe_version(void);

/* ---------------------------------------------------------------- weights ----
 * Quantize and pack one full-precision weight matrix (host memory, synchronous).
 * Follows the DeepRead summary, "Method" (weights amplified by the smoothing
 * factors) with per-output-channel symmetric round-to-nearest-even:
 *   W'[i][j] = W_f[i][j] * s[j]           (float32; s == NULL means s = 1)
 *   w_scale[i] = max_j |W'[i][j]| / qmax    (qmax = 7 for w_bits 4, 3 for w_bits 3)
 *   q[i][j] = clamp(rint(W'[i][j] / w_scale[i]), -qmax, qmax); all-zero rows -> 0
 * Packed layouts (canonical, two's complement):
 *   w_bits 4: uint8 [d_out][d_in/2]; byte m holds code 2m in bits 0-3, 2m+1 in bits 4-7.
 *   w_bits 3: uint32 [d_out][d_in/32][3]; 32 codes per 96-bit little-endian group,
 *             code c at bits 3c..3c+2.
 * W_f_host: float32 [d_out][d_in]; s_host: float32 [d_in] or NULL;
 * packed_host: d_out*d_in/2 bytes (W4) or d_out*d_in*3/8 bytes (W3);
 * w_scale_host: float32 [d_out].  Requires d_in even (W4) or d_in % 32 == 0 (W3).
 */
int qe_pack_weights(const float* W_f_host, const float* s_host, int32_t d_out, int32_t d_in,
                    int32_t w_bits, void* packed_host, float* w_scale_host);

/* Bytes of the prepared parameter buffer for this linear (lin->prep ignored).  A sizing call
 * for qe_prepare's load-time layout; no step of the method. */
size_t qe_prepared_bytes(const qe_linear* lin);

/* Lay out one linear's parameters for the kernels (load-time step, enqueued on
 * `stream`): the quantized weights of the listing's W4/W3 settings (thelatestinai.com listing,
 * Tables 1-2) with the smoothing the DeepRead summary's "Method" applies before activation
 * quantization, the shared and routed adapters and the router of the same section.  A layout
 * change only; the values are those of the canonical inputs.  All inputs are device pointers in
 * the canonical layouts:
 *   w_packed  W4/W3 packed codes as produced by qe_pack_weights
 *   w_scale   float32 [d_out]
 *   smooth    float32 [d_in], entries > 0, or NULL (identity); must be NULL when a_bits == 16
 *   A_s [d_in][r_shared], B_s [r_shared][d_out]          bf16 (NULL iff r_shared == 0)
 *   A_r [n_routed][d_in][r_routed], B_r [n_routed][r_routed][d_out]  bf16
 *   R   [d_in][n_routed]                                  bf16 (NULL iff n_routed == 0)
 * prep: device output buffer of qe_prepared_bytes(lin) bytes; it becomes lin->prep.
 * The inputs may be freed once the enqueued work has finished.
 */
int qe_prepare(const qe_linear* lin, const void* w_packed, const float* w_scale, const float* smooth,
               const uint16_t* A_s, const uint16_t* B_s, const uint16_t* A_r, const uint16_t* B_r,
               const uint16_t* R, void* prep, void* stream);

/* Workspace bytes needed by qe_linear_forward / qe_route / qe_adapter_inputs /
 * qe_wq_gemm / qe_routed_lora for T tokens (the largest of them).  A sizing call; no step of
 * the method. */
size_t qe_workspace_bytes(const qe_linear* lin, int32_t T);

/* ------------------------------------------------------------ hot-path steps -- */

/* (a1) Smoothing and per-token symmetric RTN of the activations.
 * DeepRead summary, "Method": channel-wise scaling divides the activations before
 * activation quantization; A6/A8 from the listing's Tables 1-3.  In float32 with
 * IEEE division and round-half-to-even:
 *   x'[t][j] = x[t][j] / s[j];  s_x[t] = max_j |x'[t][j]| / qmax  (qmax 31 or 127)
 *   codes[t][j] = clamp(rint(x'[t][j] / s_x[t]), -qmax, qmax); all-zero token -> 0
 * x: device [T][d_in] (x_dtype); smooth: device [d_in] or NULL (identity);
 * codes: device int8 [T][d_in]; s_x: device float32 [T].  a_bits 6 or 8; d_in % 8 == 0 and
 * d_in <= 32768 (else QE_ERR_UNSUPPORTED).
 */
int qe_quant_act(const void* x, int32_t x_dtype, const float* smooth, int32_t T, int32_t d_in,
                 int32_t a_bits, int8_t* codes, float* s_x, void* stream);

/* (a5) Router and token bucketing.
 * DeepRead summary, "Method" (router picks the routed expert with the smallest
 * predicted error) and the listing's Table 7 (one d x N_r map per token):
 *   scores[t][e] = sum_j bf16(x)[t][j] * R[j][e]  (float32 accumulation of exact products)
 *   expert[t] = argmin_e scores[t][e], lowest e on ties
 *   counts[e] = #tokens routed to e; offsets = exclusive prefix sum (offsets[N_r] = T);
 *   perm = token indices sorted by (expert, token index)
 * x: device [T][d_in]; scores: device float32 [T][n_routed] or NULL;
 * expert, perm: device int32 [T]; counts: int32 [n_routed]; offsets: int32 [n_routed+1].
 * Requires lin->n_routed > 0.  ws: workspace of ws_bytes >= qe_workspace_bytes(lin, T).
 */
int qe_route(const qe_linear* lin, const void* x, int32_t x_dtype, int32_t T, float* scores,
             int32_t* expert, int32_t* counts, int32_t* offsets, int32_t* perm,
             void* ws, size_t ws_bytes, void* stream);

/* (a4/a6, first half) Adapter inputs: u = bf16(x) . A_s and v[t] = bf16(x)[t] . A_{expert[t]},
 * accumulated in float32 and stored as bf16 (round to nearest even).
 * DeepRead summary, "Method": the shared expert and each routed expert are low-rank
 * adapters on the layer input; the listing's Table 7 counts d*r multiply-adds per token for
 * each (dense over all input channels), which is this projection plus the second half.
 * Adapter-input rows are padded to whole bf16 MFMA steps: u is device bf16 [T][ru] with
 * ru = r_shared rounded up to a multiple of 32, v is [T][rv] with rv = r_routed rounded up
 * to a multiple of 32; the padding columns are written as zeros.
 * u: NULL iff r_shared == 0; v and expert (device int32 [T], values in [0, n_routed)):
 * NULL iff n_routed == 0.
 */
int qe_adapter_inputs(const qe_linear* lin, const void* x, int32_t x_dtype, int32_t T,
                      const int32_t* expert, uint16_t* u, uint16_t* v,
                      void* ws, size_t ws_bytes, void* stream);

/* (a3, plus the second halves of a4/a6; a7 when a_bits == 16) Quantized main
 * product with a float32 dequantization epilogue into which the shared and the
 * selected routed low-rank terms are fused (listing, Table 7: the s*d^2 term):
 *   a_bits 6/8: acc[t][i] = sum_j codes[t][j] * q_w[i][j]   (exact int32)
 *               y[t][i] = acc * s_x[t] * w_scale[i] + u[t].B_s[:,i] + v[t].B_{expert[t]}[:,i]
 *   a_bits 16:  y[t][i] = w_scale[i] * sum_j bf16(x)[t][j] * q_w[i][j] + (same adapter terms)
 * codes/s_x: from qe_quant_act (a_bits 6/8; NULL for 16); x: device [T][d_in] (a_bits 16 only,
 * else ignored); u, v, expert as produced by qe_adapter_inputs / qe_route (u NULL => no shared
 * term; v and expert both NULL => no routed term); perm: device int32 [T] or NULL, a
 * permutation of the tokens (e.g. qe_route's, grouped by expert) in which the kernel visits
 * them -- it changes only the schedule, not the result; ignored for a_bits 16.
 * y: device float32 [T][d_out], overwritten; acc_debug: device int32 [T][d_out] or NULL
 * (a_bits 6/8 only).
 */
int qe_wq_gemm(const qe_linear* lin, const int8_t* codes, const float* s_x, const void* x,
               int32_t x_dtype, int32_t T, const uint16_t* u, const uint16_t* v,
               const int32_t* expert, const int32_t* perm, float* y, int32_t* acc_debug,
               void* ws, size_t ws_bytes, void* stream);

/* (a6, unfused form) Routed experts as a grouped low-rank product over the
 * expert buckets: for each expert e and each token t in perm[offsets[e]..offsets[e+1]):
 *   y[t] += (bf16(x)[t] . A_e) . B_e      (y is ADDED to, not overwritten)
 * DeepRead summary, "Method", Routed Experts: each token uses the one routed low-rank
 * adapter its router picked; PaperDaily post "核心设计": the compensations are added.
 * expert/offsets/perm as produced by qe_route.
 */
int qe_routed_lora(const qe_linear* lin, const void* x, int32_t x_dtype, int32_t T,
                   const int32_t* expert, const int32_t* offsets, const int32_t* perm, float* y,
                   void* ws, size_t ws_bytes, void* stream);

/* The activation-side half of the QE linear, fused: one pass of the x-projection gives the
 * router scores (a5) and both adapter inputs (a4/a6 first halves), then the per-token
 * quantization (a1).  DeepRead summary, "Method": smoothing and activation quantization
 * (Shared Expert paragraph), the router that picks the expert with the smallest predicted
 * error and the adapters on the layer input (Routed Experts paragraph).  Equivalent to qe_route + qe_adapter_inputs + qe_quant_act, with one
 * read of x for all projections.  Outputs (device, caller-owned): codes int8 [T][d_in] and
 * s_x float32 [T] (a_bits 6/8; both NULL for a_bits 16), u and v as for
 * qe_adapter_inputs (padded rows), expert int32 [T], and perm int32 [T] or NULL (tokens
 * sorted by (expert, token), as qe_route's).  Feed them to qe_wq_gemm.  With bf16 x and more
 * than 16 tokens it runs as two reads of x (scores, u and max |x/s|; then codes and v), or,
 * for up to 128 tokens (256 without a shared expert) and d_in <= 8192, as one launch with a
 * workgroup per token.  Codes and s_x do not depend on the form; the float32 sums behind the
 * scores, u and v are added in another order (routes can differ only at near-ties).
 */
int qe_linear_prologue(const qe_linear* lin, const void* x, int32_t x_dtype, int32_t T, int8_t* codes,
                       float* s_x, uint16_t* u, uint16_t* v, int32_t* expert, int32_t* perm,
                       void* ws, size_t ws_bytes, void* stream);

/* The whole QE linear: qe_linear_prologue followed by qe_wq_gemm (a1 + a5 + a4 + a6 + a3,
 * or a7 for a_bits 16).  DeepRead summary, "Method": every token uses the quantized layer,
 * the fixed shared expert and one routed expert chosen by the router; PaperDaily post
 * "核心设计": the three results are summed; listing, Table 7: the cost s*d^2 + s*d*(2r + N_r).  y: device float32 [T][d_out] (overwritten); expert_out: device int32 [T]
 * or NULL (the routed expert of each token).  ws: qe_workspace_bytes(lin, T) bytes.
 */
int qe_linear_forward(const qe_linear* lin, const void* x, int32_t x_dtype, int32_t T, float* y,
                      int32_t* expert_out, void* ws, size_t ws_bytes, void* stream);

/* Linears that read the same input (q, k and v of an attention block; gate and up of an MLP):
 * the QE linear of each (DeepRead summary, "Method"), with the input read once for all of their
 * route passes (and, when every linear is routed with the same rank, one launch per step for the
 * rest of their prologues).  lins[0..n_lin) (1 <= n_lin <= 3, equal d_in); x as for qe_linear_forward;
 * every other pointer argument is an array of n_lin entries, entry i meaning what the same
 * argument of qe_linear_prologue / qe_linear_forward means for lins[i]; ws[i] holds
 * ws_bytes[i] >= qe_workspace_bytes(lins[i], T) bytes, one workspace per linear.  Results are
 * identical, bit for bit, to calling qe_linear_prologue / qe_linear_forward on each linear in
 * turn, which is what happens when the group cannot share the pass (fewer than 2 linears,
 * float32 x, 16 tokens or fewer, weight-only linears, more than 48 projected columns, or few
 * enough tokens for each linear's one-launch prologue: see qe_linear_prologue).
 * Errors as for the single-linear calls; any invalid entry fails the whole call before any
 * launch.
 */
int qe_group_prologue(const qe_linear* const* lins, int32_t n_lin, const void* x, int32_t x_dtype, int32_t T,
                      int8_t* const* codes, float* const* s_x, uint16_t* const* u, uint16_t* const* v,
                      int32_t* const* expert, int32_t* const* perm, void* const* ws, const size_t* ws_bytes,
                      void* stream);
int qe_group_forward(const qe_linear* const* lins, int32_t n_lin, const void* x, int32_t x_dtype, int32_t T,
                     float* const* y, int32_t* const* expert_out, void* const* ws, const size_t* ws_bytes,
                     void* stream);
/* The main products of a group (qe_wq_gemm for each linear, a_bits 6/8 only; the quantized
 * product with the fused adapter terms of the listing's Table 7 and the DeepRead summary's
 * "Method", as for qe_wq_gemm): when every linear takes the fast path without a K split
 * (float32 y, ranks <= 32) and every linear's tile grid is a multiple of 8 workgroups, one
 * launch runs all of them, so narrow projections (k, v) share the grid of a wide one (q) instead
 * of running a grid of their own: 128-token tiles when the combined grid of those is at least
 * 512 workgroups, else 64-token tiles; otherwise one product after the other.  Identical results
 * either way.  Arrays of n_lin entries as for qe_group_prologue (its
 * outputs are this call's inputs); qe_group_forward ends with this step.
 */
int qe_group_gemm(const qe_linear* const* lins, int32_t n_lin, const int8_t* const* codes, const float* const* s_x,
                  int32_t T, const uint16_t* const* u, const uint16_t* const* v, const int32_t* const* expert,
                  const int32_t* const* perm, float* const* y, void* const* ws, const size_t* ws_bytes, void* stream);

/* For callers that cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): qe_linear_forward without a workspace argument.  It
 * computes exactly what qe_linear_forward computes (the same kernels), with its workspace in a
 * file-scope device array of qe_noalloc_scratch_bytes() bytes (64 MiB) that each GPU holds from
 * the library's first use on it until the process ends; its device address is looked up once
 * per device on the first call made with that device current.  The call itself allocates
 * nothing.  Calls with qe_workspace_bytes(lin, T) > qe_noalloc_scratch_bytes() return
 * QE_ERR_WORKSPACE and launch nothing (the decode and few-token calls of the 72B-wide linears
 * fit; whole 4096-token prefills of them do not).  Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (different streams, or threads without ordering) race
 * and give undefined results; calls ordered on one stream are safe.  The array keeps the last
 * call's contents; every value the kernels read from it is written earlier in the same call.
 * Other arguments, errors and output as for qe_linear_forward.
 */
size_t qe_noalloc_scratch_bytes(void);
int qe_linear_forward_noalloc(const qe_linear* lin, const void* x, int32_t x_dtype, int32_t T, float* y,
                              int32_t* expert_out, void* stream);

/* ------------------------------------------------- channel-importance statistic --
 * (a8 helper) w[j] = (sum_i |W[i][j]|) / d_out: the column mean of |W_f|, one value
 * per input channel (DeepRead summary, "Method", first paragraph: Mean_row(|W_f|)).
 * Summed in float64 and rounded once to float32.  W: device [d_out][d_in] (dtype);
 * w: device float32 [d_in].
 */
int qe_colmean_abs(const void* W, int32_t dtype, int32_t d_out, int32_t d_in, float* w, void* stream);

/* (a8) Per-token important channels and their frequency (DeepRead summary,
 * "Method": S_t = Top-k(|x_t| * w); the listing's Figure 3 counts how often each
 * channel is selected):
 *   sc[t][j] = |x[t][j]| * w[j]  (float32, x at its stored precision)
 *   topk[t][0..k) = the k channels first in the order (sc descending, j ascending)
 *   hist[j] += #{t : j in topk[t]}   (hist is ACCUMULATED; the caller zeroes it)
 * x: device [T][d_in]; w: device float32 [d_in] (entries >= 0);
 * topk: device int32 [T][k] or NULL; hist: device uint32 [d_in].  1 <= k <= min(d_in, 1024),
 * d_in <= 32768.
 */
int qe_channel_topk(const void* x, int32_t x_dtype, const float* w, int32_t T, int32_t d_in,
                    int32_t k, int32_t* topk, uint32_t* hist, void* stream);

/* ------------------------------------------ channel partition and clustering --
 * The rest of the calibration statistic (DeepRead summary, "Method": channels ordered
 * by selection frequency, the first k token-independent and the next N_r * k
 * token-dependent; the token-dependent channels grouped into N_r clusters by spectral
 * clustering of their NPMI co-occurrence similarity; PaperDaily post, "核心设计":
 * O[t][i], the co-occurrence counts, p(i), p(i,j), NPMI and its threshold; listing,
 * Figure 6).
 *
 * qe_partition_channels (host, synchronous): orders the channels by hist descending,
 *   ties by ascending channel index, and writes indep[0..k) = the first k and
 *   dep[0..n_r*k) = the next n_r*k.  slot (optional) receives, for every channel, its
 *   position in dep or -1.  hist: host uint32 [d_in] (qe_channel_topk's histogram copied
 *   to the host); indep, dep, slot: host int32 buffers of k, n_r*k and d_in entries.
 *   Requires k >= 1, n_r >= 1, k * (1 + n_r) <= d_in.
 */
int qe_partition_channels(const uint32_t* hist, int32_t d_in, int32_t k, int32_t n_r, int32_t* indep,
                          int32_t* dep, int32_t* slot);

/* qe_cooccur (device; DeepRead summary, "Method", and the PaperDaily post "西交大提出Quant
 * Experts：token级量化补偿", section "核心设计": the co-occurrence matrix of the token-dependent
 * channels): cooc[i][j] += #{t : topk[t] holds both dep[i] and dep[j]}, i.e.
 *   cooc += O^T O with O[t][i] = 1 when token t selected the i-th token-dependent channel.
 *   The diagonal counts each channel's selections.  cooc is ACCUMULATED over calls (the
 *   caller zeroes it), so a calibration set can be fed in batches of tokens.
 *   topk: device int32 [T][k] as written by qe_channel_topk (each row a set of distinct
 *   channels); slot: device int32 [d_in] as written by qe_partition_channels (entries
 *   outside [0, n_dep) mark channels that are not token-dependent; topk entries outside
 *   [0, d_in) are skipped); cooc: device uint32 [n_dep][n_dep]; ws: device scratch of
 *   ws_bytes >= qe_cooccur_workspace_bytes(T, n_dep) (the per-token channel bit masks;
 *   contents on entry do not matter, else QE_ERR_WORKSPACE).  All 16-byte aligned.
 *   1 <= k <= min(d_in, 1024); 1 <= n_dep <= 8192.  T == 0 is a no-op.
 * qe_cooccur_workspace_bytes: scratch bytes for T tokens (0 for invalid sizes); enough for
 *   any call with at most T tokens.
 */
size_t qe_cooccur_workspace_bytes(int32_t T, int32_t n_dep);
int qe_cooccur(const int32_t* topk, int32_t T, int32_t k, const int32_t* slot, int32_t d_in, int32_t n_dep,
               uint32_t* cooc, void* ws, size_t ws_bytes, void* stream);

/* qe_cluster_channels (host, synchronous; DeepRead summary, "Method": NPMI similarity, spectral
 *   clustering of the normalized Laplacian and K-Means into N_r clusters; PaperDaily post, section
 *   "核心设计": p(i), p(i,j), the threshold): from the co-occurrence counts of n_dep
 *   token-dependent channels over T tokens,
 *     NPMI(i,j) = ln(p_ij / (p_i p_j)) / -ln p_ij,  p_ij = cooc[i][j] / T, p_i = cooc[i][i] / T,
 *     with -1 where p_ij = 0 and +1 where p_ij = 1;
 *     S[i][j] = NPMI(i,j) if NPMI(i,j) >= threshold, else 0;
 *     L = I - D^-1/2 S D^-1/2 (d_i = sum_j S[i][j]; rows with d_i = 0 contribute nothing);
 *     U = eigenvectors of the n_clusters smallest eigenvalues of L, rows scaled to unit
 *     length (Ng, Jordan and Weiss); labels = K-Means of the rows of U (Lloyd's iteration
 *     from farthest-point seeds starting at row 0; ties to the lower index), numbered in
 *     order of each cluster's lowest member.
 *   cooc: host uint32 [n_dep][n_dep] (qe_cooccur's result copied to the host; symmetric,
 *   cooc[i][j] <= min(cooc[i][i], cooc[j][j]), cooc[i][i] <= T, else QE_ERR_INVALID_ARG);
 *   labels: host int32 [n_dep]; similarity (host double [n_dep][n_dep]), eigvals (host
 *   double [n_clusters], ascending) and embedding (host double [n_dep][n_clusters]) are
 *   optional outputs (NULL to skip).  1 <= n_clusters <= n_dep <= 2048; T >= 1;
 *   0 <= threshold <= 1.  Returns QE_ERR_UNSUPPORTED if the eigenvalue iteration does not
 *   converge.
 */
int qe_cluster_channels(const uint32_t* cooc, int32_t n_dep, int64_t T, int32_t n_clusters, double threshold,
                        int32_t* labels, double* similarity, double* eigvals, double* embedding);

/* ----------------------------------------------------------------- accounting --
 * Algorithmic work of one QE linear over T tokens (listing, Table 7, generalised
 * to d_in != d_out):
 *   int_macs      = T * d_in * d_out                        (the quantized product)
 *   adapter_macs  = T * (d_in + d_out) * (r_shared + r_routed) + T * d_in * n_routed
 *   alg_bytes     = minimum HBM traffic: x read once, packed weights, scales, y written
 *                   once (4 or 2 bytes per element as y_dtype says), A_s, B_s, R and the A_e, B_e of n_distinct_experts
 *                   distinct routed experts actually selected.
 * Host-only; x_bytes_per_elt is 2 (bf16) or 4 (float32).
 */
int qe_linear_cost(const qe_linear* lin, int32_t T, int32_t n_distinct_experts, int32_t x_bytes_per_elt,
                   double* int_macs, double* adapter_macs, double* alg_bytes);

/* Top-2 routing (PaperDaily post "西交大提出Quant Experts：token级量化补偿", section "核心设计":
 * at inference only the top-1 or the top-2 routed experts are activated).  The token takes the
 * two experts with the smallest router scores (the lower index on ties) and both routed
 * corrections are added: each routed expert is fitted to the error of its own cluster of
 * channels, so the two corrections are complementary (the pages give no combining rule).
 * qe_linear_forward_top2: y as qe_linear_forward plus (x A_e2) B_e2 for the second expert e2 =
 *   the smallest score among the experts other than the forward's first expert (both taken
 *   from the same router scores where the main product runs unsplit on 128-token tiles, which
 *   then adds both corrections in its epilogue).  Requires n_routed >= 2, T <= 65535.
 *   expert_out / expert2_out: optional device int32 [T].  ws: qe_top2_workspace_bytes(lin, T)
 *   bytes (qe_workspace_bytes' layout plus the routes, scores, the second expert's grouping
 *   and its adapter input).  Enqueued; errors as qe_linear_forward.
 */
size_t qe_top2_workspace_bytes(const qe_linear* lin, int32_t T);
int qe_linear_forward_top2(const qe_linear* lin, const void* x, int32_t x_dtype, int32_t T, float* y,
                           int32_t* expert_out, int32_t* expert2_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------- expert construction --
 * Building the shared and routed experts of one linear after calibration (MCISLAB DeepRead
 * summary of "Quant Experts", section "Method": the quantization error E = W_f - W_q is
 * reconstructed by the low-rank shared expert, the error left after it by one low-rank
 * routed expert per cluster of token-dependent channels; PaperDaily post "西交大提出Quant
 * Experts：token级量化补偿", section "核心设计": by a whitening SVD).  The whitening is
 * diagonal, with the RMS of each input channel's calibration activations; the truncated SVD
 * is the randomized subspace iteration of Halko, Martinsson and Tropp ("Finding structure with
 * randomness", Algorithms 4.4 and 5.1) with the Gaussian test matrix supplied by the caller.
 * The router fit is by ridge least squares on per-token targets (below).
 *
 * qe_quant_error: E = W_f - diag(s_w) q diag(1/s) (float32, device [d_out][d_in]) with the
 *   codes and row scales qe_pack_weights takes (same float32 arithmetic).  W_f device float32
 *   [d_out][d_in]; s device float32 [d_in] or NULL; w_bits 3 or 4.  Enqueued on `stream`.
 * qe_channel_rms: c[j] = sqrt(mean_t x[t][j]^2) over T calibration tokens (x device
 *   [T][d_in], QE_F32 or QE_BF16; c device float32 [d_in]; sums in double).  ws: device,
 *   qe_channel_rms_workspace_bytes(T, d_in) bytes.  Enqueued.
 * qe_sub_lowrank: E[i][j] -= sum_l A[j][l] B[l][i] in place (A device float32 [d_in][r], B
 *   device float32 [r][d_out], 1 <= r <= 64).  Enqueued.
 * qe_lowrank_fit: rank-`rank` factors of M = diag(w) E^T (w device float32 [d_in], entries >= 0,
 *   or NULL for ones; E device float32 [d_out][d_in]); omega device float32 [d_out][k], the
 *   test matrix (Gaussian entries); 1 <= rank <= k <= min(128, d_in, d_out); 0 <= power_iters
 *   <= 16.  Outputs on the HOST: A float32 [d_in][rank] = diag(1/w) U_r S_r^(1/2) (rows with
 *   w = 0 are zero), B float32 [rank][d_out] = S_r^(1/2) V_r^T, sigma double [rank] (descending).
 *   ws: device, qe_lowrank_workspace_bytes(d_out, d_in, k) bytes.  Synchronizes `stream`: the
 *   passes over E, the k x k Gram matrices (double sums) and the products with k x k matrices
 *   run on the GPU; the k x k eigenproblems that orthonormalize (twice, by the Gram matrix;
 *   directions below 1e-11 of its largest eigenvalue dropped as null) run on the host.
 * qe_build_experts: the whole construction for one linear: E = qe_quant_error(W_f, s); the SE
 *   (rank r_shared, 0 = none) = qe_lowrank_fit(E, c, omegas[0]); E_1 = E - (A_s B_s)^T; for each
 *   routed expert g < n_routed (<= 16): qe_lowrank_fit(E_1, c on the channels dep_channels[t]
 *   with labels[t] == g and 0 elsewhere, omegas[1 + g]) with rank r_routed (1..64; ignored when
 *   n_routed == 0).  c: device float32 [d_in] (qe_channel_rms); dep_channels, labels: HOST int32
 *   [n_dep] (channel ids in [0, d_in), cluster ids in [0, n_routed), e.g. from
 *   qe_partition_channels and qe_cluster_channels); omegas: device float32 [1 + n_routed][d_out][k]
 *   (entry 0 unused when r_shared == 0).  Outputs on the HOST, float32: A_s [d_in][r_shared],
 *   B_s [r_shared][d_out], A_r [n_routed][d_in][r_routed], B_r [n_routed][r_routed][d_out];
 *   sigma_s [r_shared], sigma_r [n_routed][r_routed] double.  ws: device,
 *   qe_build_experts_workspace_bytes(d_out, d_in, k, max(r_shared, r_routed)) bytes (it holds E).
 *   Synchronizes `stream`.
 * Errors: QE_ERR_INVALID_ARG / QE_ERR_ALIGNMENT / QE_ERR_WORKSPACE before any work;
 * QE_ERR_UNSUPPORTED if the small eigenvalue iteration fails to converge; QE_ERR_HIP.
 */
int qe_quant_error(const float* W_f, const float* s, int32_t d_out, int32_t d_in, int32_t w_bits, float* E,
                   void* stream);
size_t qe_channel_rms_workspace_bytes(int32_t T, int32_t d_in);
int qe_channel_rms(const void* x, int32_t x_dtype, int32_t T, int32_t d_in, float* c, void* ws, size_t ws_bytes,
                   void* stream);
int qe_sub_lowrank(float* E, int32_t d_out, int32_t d_in, const float* A, const float* B, int32_t r, void* stream);
size_t qe_lowrank_workspace_bytes(int32_t d_out, int32_t d_in, int32_t k);
int qe_lowrank_fit(const float* E, int32_t d_out, int32_t d_in, const float* w, const float* omega, int32_t k,
                   int32_t rank, int32_t power_iters, float* A, float* B, double* sigma, void* ws, size_t ws_bytes,
                   void* stream);
size_t qe_build_experts_workspace_bytes(int32_t d_out, int32_t d_in, int32_t k, int32_t r_max);
int qe_build_experts(const float* W_f, const float* s, int32_t d_out, int32_t d_in, int32_t w_bits, const float* c,
                     const int32_t* dep_channels, const int32_t* labels, int32_t n_dep, int32_t n_routed,
                     int32_t r_shared, int32_t r_routed, const float* omegas, int32_t k, int32_t power_iters,
                     float* A_s, float* B_s, float* A_r, float* B_r, double* sigma_s, double* sigma_r, void* ws,
                     size_t ws_bytes, void* stream);

/* Expert construction by covariance whitening (the default construction).  PaperDaily post
 * "西交大提出Quant Experts：token级量化补偿", section "核心设计": the error minus the shared and
 * routed compensations, multiplied by the input token, is to leave the smallest residual, and
 * the whitening SVD computes a covariance and whitens with it.  Reading: the SE of rank r is
 * the minimizer of sum_t |(E - A_hat) x_t|^2 over the calibration tokens, i.e. A_hat =
 * U_r U_r^T E with U_r the top-r eigenvectors of the error-output covariance
 * C = sum_t (E x_t)(E x_t)^T (Eckart-Young on Z = E X^T; the same subspace as the SVD of E L
 * with L L^T = X^T X); the RE of cluster g is the same fit of the residual E_1 = E - A_hat_s
 * restricted to the cluster's input channels (DeepRead summary, "Method": the error left after
 * the SE goes to one routed expert per cluster).  The top-r vectors come from the randomized
 * subspace iteration (Halko, Martinsson and Tropp, Algorithms 4.4 and 5.1) on the operator Z,
 * applied by passes over E and X; Z and C are never formed.
 * qe_lowrank_fit_cov: factors of E diag(mask) for tokens X (device float32 [T][d_in]); mask
 *   device float32 [d_in] of 0/1 or NULL (all channels); E device float32 [d_out][d_in];
 *   omega device float32 [T][k] (Gaussian entries); 1 <= rank <= k <= min(128, d_out, T);
 *   0 <= power_iters <= 16.  Outputs on the HOST: A float32 [d_in][rank] = diag(mask) E^T U_r,
 *   B float32 [rank][d_out] = U_r^T (so x A B = x A_hat^T), sigma double [rank] = the top
 *   singular values of Z (descending; directions below 1e-11 of the largest eigenvalue are
 *   dropped: zero sigma and zero columns).  ws: device, qe_lowrank_cov_workspace_bytes(d_out,
 *   d_in, T, k) bytes.  Synchronizes `stream`.
 * qe_build_experts_cov: E = qe_quant_error(W_f, s); the SE (rank r_shared, 0 = none) =
 *   qe_lowrank_fit_cov(E, all channels, omegas[0]); E_1 = E - (A_s B_s)^T; routed expert g <
 *   n_routed (<= 16): qe_lowrank_fit_cov(E_1, mask of the channels dep_channels[t] with
 *   labels[t] == g, omegas[1 + g]), rank r_routed (1..64).  x: device [T][d_in] calibration
 *   tokens (QE_F32 or QE_BF16; the layer input the adapters read); omegas device float32
 *   [1 + n_routed][T][k]; dep_channels, labels HOST int32 [n_dep].  Outputs on the HOST as for
 *   qe_build_experts.  ws: device, qe_build_experts_cov_workspace_bytes(d_out, d_in, T, k,
 *   max(r_shared, r_routed)) bytes (it holds E and a float32 copy of x).  Synchronizes `stream`.
 * Errors: QE_ERR_INVALID_ARG / QE_ERR_ALIGNMENT / QE_ERR_WORKSPACE before any work;
 * QE_ERR_UNSUPPORTED if the small eigenvalue iteration fails to converge; QE_ERR_HIP.
 */
size_t qe_lowrank_cov_workspace_bytes(int32_t d_out, int32_t d_in, int32_t T, int32_t k);
int qe_lowrank_fit_cov(const float* E, int32_t d_out, int32_t d_in, const float* X, int32_t T, const float* mask,
                       const float* omega, int32_t k, int32_t rank, int32_t power_iters, float* A, float* B,
                       double* sigma, void* ws, size_t ws_bytes, void* stream);
size_t qe_build_experts_cov_workspace_bytes(int32_t d_out, int32_t d_in, int32_t T, int32_t k, int32_t r_max);
int qe_build_experts_cov(const float* W_f, const float* s, int32_t d_out, int32_t d_in, int32_t w_bits,
                         const void* x, int32_t x_dtype, int32_t T, const int32_t* dep_channels,
                         const int32_t* labels, int32_t n_dep, int32_t n_routed, int32_t r_shared, int32_t r_routed,
                         const float* omegas, int32_t k, int32_t power_iters, float* A_s, float* B_s, float* A_r,
                         float* B_r, double* sigma_s, double* sigma_r, void* ws, size_t ws_bytes, void* stream);

/* Router fit (MCISLAB DeepRead summary, "Method", Routed Experts: the router estimates the error
 * each routed expert would leave on a token and the token takes the smallest; WisPaper post
 * "[CVPR 2025] Quant Experts: Adapting PTQ to the Heterogeneity of Vision-Language Tokens",
 * section "Critical Analysis & Insight": an absolute mean error prediction).
 * qe_router_targets: target[t][g] = mean_i |x_t (E_1^T - A_g B_g)|_i over the d_out outputs for
 *   T calibration tokens x (device [T][d_in], QE_F32 or QE_BF16); E_1 device float32 [d_out][d_in]
 *   (the error left after the shared expert); A_r device float32 [n_routed][d_in][r_routed], B_r
 *   [n_routed][r_routed][d_out] (n_routed <= 16, r_routed <= 64); target device float32
 *   [T][n_routed].  ws: device, qe_router_targets_workspace_bytes(...) bytes.  Enqueued.
 * qe_router_fit: R = argmin |X R - target|^2 + lam |R|^2 with lam = ridge * |X|_F^2 / d_in, by
 *   conjugate gradients on (X^T X + lam I) R = X^T target (one system per column), until every
 *   column's residual is below tol times its right-hand side or after max_iters iterations.
 *   x device [T][d_in] (QE_F32 / QE_BF16), target device float32 [T][n_routed]; R HOST float32
 *   [d_in][n_routed] (the router, to be given to qe_prepare in bf16); *iters_done (optional)
 *   receives the iterations taken.  ws: device, qe_router_fit_workspace_bytes(T, d_in, n_routed)
 *   bytes (it holds a float32 copy of x).  Synchronizes `stream`.
 */
size_t qe_router_targets_workspace_bytes(int32_t d_out, int32_t d_in, int32_t n_routed, int32_t r_routed);
int qe_router_targets(const float* E1, int32_t d_out, int32_t d_in, const void* x, int32_t x_dtype, int32_t T,
                      const float* A_r, const float* B_r, int32_t n_routed, int32_t r_routed, float* target, void* ws,
                      size_t ws_bytes, void* stream);
size_t qe_router_fit_workspace_bytes(int32_t T, int32_t d_in, int32_t n_routed);
int qe_router_fit(const void* x, int32_t x_dtype, int32_t T, int32_t d_in, const float* target, int32_t n_routed,
                  double ridge, int32_t max_iters, double tol, float* R, int32_t* iters_done, void* ws, size_t ws_bytes,
                  void* stream);

/* ---------------------------------------------------------- measurement aids --
 * Not part of the QE computation: kernels whose duration, measured by the caller with
 * events on `stream`, gives the rates this device sustains, reported beside the
 * published peaks when the hot path's kernels are placed on their roofline.
 *
 * qe_probe_mfma_i8: `blocks` workgroups of 256 threads (blocks >= 1); each of their waves
 *   issues 8 * iters int8 16x16x64 MFMAs (the main GEMM's instruction) into 8 independent
 *   accumulators, on register operands fixed through the loop.  The matrix cores are
 *   power-limited, so the rate depends on the values: operands = 0 uses small constant
 *   bytes (the highest rate the part sustains), operands = 1 random values in the main
 *   GEMM's ranges (A6 codes in [-31, 31] times 4-bit codes scaled by 16).  *ops receives
 *   the integer operations enqueued (2 * 16 * 16 * 64 per MFMA).  out: device int32
 *   [blocks * 256 * 4], a result sink the caller owns.  iters >= 1.
 * qe_probe_mfma_bf16: the same loop on bf16 16x16x32 MFMAs (the weight-only GEMM's
 *   instruction) with float32 accumulators: operands = 0 small constants, operands = 1
 *   random values in that GEMM's ranges (activations of unit scale, 3-bit codes times a
 *   scale near 2^-7).  *flops receives 2 * 16 * 16 * 32 per MFMA.  out: device float32
 *   [blocks * 256 * 4], a result sink the caller owns.
 * qe_probe_copy: copies `bytes` (a multiple of 16) from src to dst; both device pointers,
 *   16-byte aligned, caller-owned, not overlapping.  The traffic is 2 * bytes.
 * qe_probe_read: reads `bytes` (a multiple of 16) from src once (device, 16-byte aligned) and
 *   writes one folded word per thread to sink (device, qe_probe_read_sink_bytes() bytes): the
 *   read-only streaming rate, for weight-streaming kernels whose traffic is almost all reads.
 * Both only enqueue work (no synchronization); invalid arguments return
 * QE_ERR_INVALID_ARG / QE_ERR_ALIGNMENT and launch nothing.
 */
int qe_probe_mfma_i8(int32_t* out, int32_t blocks, int32_t iters, int32_t operands, double* ops, void* stream);
int qe_probe_mfma_bf16(float* out, int32_t blocks, int32_t iters, int32_t operands, double* flops, void* stream);
int qe_probe_copy(const void* src, void* dst, size_t bytes, void* stream);
size_t qe_probe_read_sink_bytes(void);
int qe_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QE_H */
