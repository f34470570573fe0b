"""CPU oracle for the Quant Experts (QE) linear-layer hot path.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, obviously correct
definition of what the hot path computes.  Only the test suite, the smoke check
of the package entry file and the CPU-baseline leg of the benchmark may import
it; the product path (the HIP library and its Python binding) never does.  It
shares no code with the HIP path.

Sources (the pages; cited by title and section):
  [DeepRead]  MCISLAB DeepRead summary "Quant Experts: Token-aware Adaptive Error
              Reconstruction with Mixture of Experts for Large Vision-Language
              Models Quantization", sections "Method" and "Strengths & Weaknesses".
  [PaperDaily] longzhangge PaperDaily post "西交大提出Quant Experts：token级量化补偿",
              sections "从观察到创新" and "核心设计".
  [wispaper]  wispaper.ai post "Quant Experts: Adapting PTQ to the Heterogeneity of
              Vision-Language Tokens", "Methodology" and "Critical Analysis".
  [listing]   thelatestinai.com listing of arXiv 2602.24059, Tables 1-13, Figures 1-6.

Precision: integer parts are exact; floating-point reductions are done in
float64 and rounded once to float32 at the output.  Where a floating-point value
decides an integer (activation/weight codes), the decision is taken in float32,
the precision the HIP kernels use, with IEEE division and round-half-to-even.

Readings of open points (each also listed in the design notes):
  * w = Mean_row(|W_f|) is the mean over output rows: one value per input channel.
  * Top-k ties go to the lower channel index; sets are ordered (score desc, index asc).
  * Activation quantization is per-token symmetric RTN with qmax = 2^(b-1)-1 after
    dividing x by the smoothing vector; weight quantization is per-output-channel
    symmetric RTN of W_f * diag(s).  An all-zero token/row has scale 0 and codes 0.
  * The shared expert, the router and the routed experts all read the layer input
    x rounded to bf16 (not smoothed, not quantized); outputs are summed in parallel.
  * The router scores each expert with one linear map x.R and picks the smallest
    score (the pages: the router predicts each expert's remaining error and picks
    the smallest); ties go to the lower expert index; one routed expert per token.

Parity-pinned: every public function below is pinned by the tests in
tests/test_oracle_*.py (brute force on tiny inputs, closed forms, special cases
and invariants).  Nothing here is "parity unpinned".
"""

from typing import Dict, Optional, Tuple

import numpy as np

QMAX_ACT = {6: 31, 8: 127}
QMAX_W = {4: 7, 3: 3}


# --------------------------------------------------------------------------- bf16
def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returned as float32 arrays whose low 16 bits are zero.  Inputs are finite.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32)


# ------------------------------------------------------------------ quantization
def quant_act(x: np.ndarray, s: Optional[np.ndarray], a_bits: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per-token symmetric RTN of the smoothed activations.

    [DeepRead] "Method", Shared Expert paragraph: channel-wise scaling lowers the
    activation magnitude (x / s) before activation quantization; the bit widths
    (A6, A8) are those of [listing] Tables 1-3.

    x: [T, d_in] float32 values (the stored activations); s: [d_in] float32 > 0 or None.
    Returns codes int8 [T, d_in] in [-qmax, qmax] and s_x float32 [T].
    """
    qmax = np.float32(QMAX_ACT[a_bits])
    x32 = np.asarray(x, dtype=np.float32)
    xs = x32 / np.asarray(s, dtype=np.float32)[None, :] if s is not None else x32.copy()
    T = xs.shape[0]
    if xs.shape[1] == 0:
        return np.zeros(xs.shape, np.int8), np.zeros(T, np.float32)
    amax = np.max(np.abs(xs), axis=1).astype(np.float32)
    s_x = (amax / qmax).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(xs / s_x[:, None])
    q = np.clip(q, -qmax, qmax)
    q[amax == 0] = 0
    return q.astype(np.int8), s_x


def quant_weights(W_f: np.ndarray, s: Optional[np.ndarray], w_bits: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per-output-channel symmetric RTN of W' = W_f * diag(s).

    [DeepRead] "Method": the weights are amplified by the same channel-wise factor
    the activations are divided by; W4 / W3 settings from [listing] Tables 1-3.

    Returns codes int8 [d_out, d_in] in [-qmax_w, qmax_w] and s_w float32 [d_out].
    """
    qmax = np.float32(QMAX_W[w_bits])
    W = np.asarray(W_f, dtype=np.float32)
    Wp = W * np.asarray(s, dtype=np.float32)[None, :] if s is not None else W.copy()
    amax = np.max(np.abs(Wp), axis=1).astype(np.float32)
    s_w = (amax / qmax).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(Wp / s_w[:, None])
    q = np.clip(q, -qmax, qmax)
    q[amax == 0] = 0
    return q.astype(np.int8), s_w


# ----------------------------------------------------------------------- packing
def pack_w4(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit two's-complement codes per byte: code 2m in bits 0-3, 2m+1 in bits 4-7."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    assert c.shape[1] % 2 == 0
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_w4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.int64)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.int64)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return np.where(out >= 8, out - 16, out).astype(np.int8)


def pack_w3(codes: np.ndarray) -> np.ndarray:
    """32 three-bit two's-complement codes per 96 bits (three little-endian uint32 words).

    Code c of a group sits at bits 3c..3c+2 of the 96-bit little-endian value.
    Returns uint32 [d_out, d_in/32, 3].
    """
    c = np.asarray(codes, dtype=np.int64)
    d_out, d_in = c.shape
    assert d_in % 32 == 0
    u = (c & 7).astype(np.uint64).reshape(d_out, d_in // 32, 32)
    lo = np.zeros(u.shape[:2], dtype=np.uint64)  # bits 0..63
    hi = np.zeros(u.shape[:2], dtype=np.uint64)  # bits 64..95
    for i in range(32):
        b = 3 * i
        v = u[:, :, i]
        if b + 3 <= 64:
            lo |= v << np.uint64(b)
        elif b >= 64:
            hi |= v << np.uint64(b - 64)
        else:  # straddles bit 64
            lo |= (v << np.uint64(b)) & np.uint64(0xFFFFFFFFFFFFFFFF)
            hi |= v >> np.uint64(64 - b)
    out = np.empty(u.shape[:2] + (3,), dtype=np.uint32)
    out[:, :, 0] = (lo & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    out[:, :, 1] = (lo >> np.uint64(32)).astype(np.uint32)
    out[:, :, 2] = hi.astype(np.uint32)
    return out


def unpack_w3(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint64)
    d_out, G, _ = p.shape
    out = np.empty((d_out, G, 32), dtype=np.int64)
    for i in range(32):
        b = 3 * i
        v = np.zeros((d_out, G), dtype=np.uint64)
        for k in range(3):  # gather the three bits one by one
            bit = b + k
            w, o = divmod(bit, 32)
            v |= ((p[:, :, w] >> np.uint64(o)) & np.uint64(1)) << np.uint64(k)
        out[:, :, i] = v.astype(np.int64)
    out = np.where(out >= 4, out - 8, out)
    return out.reshape(d_out, G * 32).astype(np.int8)


# -------------------------------------------------------------------- main term
def main_term_int(qx: np.ndarray, s_x: np.ndarray, qw: np.ndarray, s_w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Quantized product y_m = (q_x . q_w^T) * s_x[t] * s_w[i].

    [listing] Table 7: the sd^2 term of a QE linear is the (quantized) dense
    product.  The integer accumulator is exact: the float64 matmul of integer codes
    stays below 2^53.  Returns (acc int64 [T, d_out], y_m float64 [T, d_out]).
    """
    acc = np.asarray(qx, dtype=np.float64) @ np.asarray(qw, dtype=np.float64).T
    acc_i = acc.astype(np.int64)
    assert np.all(np.abs(acc_i) < 2**31)
    y = acc * np.asarray(s_x, np.float64)[:, None] * np.asarray(s_w, np.float64)[None, :]
    return acc_i, y


def main_term_a16(xb: np.ndarray, qw: np.ndarray, s_w: np.ndarray) -> np.ndarray:
    """Weight-only (A16) product: y_m[t, i] = s_w[i] * sum_j bf16(x)[t, j] * q_w[i, j]."""
    acc = np.asarray(xb, dtype=np.float64) @ np.asarray(qw, dtype=np.float64).T
    return acc * np.asarray(s_w, np.float64)[None, :]


# --------------------------------------------------------------------- adapters
def lowrank(xb: np.ndarray, A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """(x . A) . B in float64 for one low-rank adapter.

    [DeepRead] "Method": each expert is a low-rank adapter; [listing] Table 7 counts
    d*r multiply-adds per token for it (dense over all input channels).
    """
    u = np.asarray(xb, np.float64) @ np.asarray(A, np.float64)
    return u @ np.asarray(B, np.float64)


def route(xb: np.ndarray, R: np.ndarray) -> Dict[str, np.ndarray]:
    """Router: score_e = x . R[:, e]; the token takes the expert with the smallest score.

    [DeepRead] "Method", Routed Experts: the router estimates each expert's
    remaining error for the token and picks the one with the smallest prediction;
    [wispaper] "Critical Analysis": the prediction is a simple error estimate;
    [listing] Table 7: the router costs s*d*N_r, i.e. one d x N_r map per token.
    Ties go to the lower expert index (np.argmin returns the first minimum).
    Bucketing: counts, exclusive offsets and the token permutation sorted by
    (expert, token index).
    """
    sc = np.asarray(xb, np.float64) @ np.asarray(R, np.float64)
    T, n_r = sc.shape
    expert = np.argmin(sc, axis=1).astype(np.int32) if n_r > 0 else np.zeros(T, np.int32)
    if n_r >= 2:
        ss = np.sort(sc, axis=1)
        margin = ss[:, 1] - ss[:, 0]
        near = np.maximum(np.abs(ss[:, 0]), np.abs(ss[:, 1]))
    else:
        margin = np.full(T, np.inf)
        near = np.zeros(T)
    counts = np.bincount(expert, minlength=n_r).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    perm = np.argsort(expert, kind="stable").astype(np.int32)
    return dict(scores=sc, expert=expert, margin=margin, margin_scale=near,
                counts=counts, offsets=offsets, perm=perm)


def routed_term(xb: np.ndarray, A_r: np.ndarray, B_r: np.ndarray, expert: np.ndarray) -> np.ndarray:
    """y_r[t] = (x_t . A_{e_t}) . B_{e_t}: the one routed expert chosen for each token."""
    T = xb.shape[0]
    d_out = B_r.shape[2] if B_r.ndim == 3 else 0
    y = np.zeros((T, d_out), np.float64)
    for e in range(A_r.shape[0]):
        rows = np.nonzero(expert == e)[0]
        if len(rows):
            y[rows] = lowrank(xb[rows], A_r[e], B_r[e])
    return y


def qe_linear(x: np.ndarray, x_is_bf16: bool, s: Optional[np.ndarray], qw: np.ndarray, s_w: np.ndarray,
              a_bits: int, A_s=None, B_s=None, A_r=None, B_r=None, R=None,
              expert_override: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """One QE linear: y = Q(x/s).Q(W s)^T + SE(x) + RE_{router(x)}(x), in parallel.

    [DeepRead] "Method": every token uses the fixed shared expert plus one routed
    expert picked by the router; [PaperDaily] "核心设计": all compensations are added.
    The composition is the parallel sum of the three terms (no term reads another).

    x: [T, d_in] float32 values of the stored activations (bf16-representable if
    x_is_bf16).  qw/s_w: weight codes and scales.  Adapters/router as float32
    arrays of bf16 values (A_s [d_in, r_s], B_s [r_s, d_out], A_r [N, d_in, r],
    B_r [N, r, d_out], R [d_in, N]); any may be None (that term is absent).
    `expert_override` replaces the router's choice (used only to re-evaluate the
    output of near-tie tokens with the other valid expert).
    Returns y float32 [T, d_out] and the intermediates.
    """
    x32 = np.asarray(x, np.float32)
    xb = x32 if x_is_bf16 else bf16_round(x32)
    out: Dict[str, np.ndarray] = {}
    if a_bits == 16:
        y = main_term_a16(xb, qw, s_w)
    else:
        qx, s_x = quant_act(x32, s, a_bits)
        acc, y = main_term_int(qx, s_x, qw, s_w)
        out.update(codes=qx, s_x=s_x, acc=acc)
    y = y.copy()
    if A_s is not None and A_s.shape[1] > 0:
        y += lowrank(xb, A_s, B_s)
    if R is not None and R.shape[1] > 0:
        r = route(xb, R)
        out.update(r)
        expert = r["expert"] if expert_override is None else np.asarray(expert_override, np.int32)
        if A_r is not None:
            y += routed_term(xb, A_r, B_r, expert)
    out["y"] = y.astype(np.float32)
    out["y64"] = y
    return out


def route_top2(xb: np.ndarray, R: np.ndarray) -> Dict[str, np.ndarray]:
    """Two routed experts per token: the smallest and the second-smallest score.

    [PaperDaily] "核心设计": at inference only the top-1 or the top-2 routed experts are
    activated.  Ties go to the lower expert index (a stable sort of the scores), so expert
    is route()'s choice and expert2 the best of the others.  margin2 is the gap between the
    second and third smallest scores (for near-tie checks).
    """
    sc = np.asarray(xb, np.float64) @ np.asarray(R, np.float64)
    T, n_r = sc.shape
    order = np.argsort(sc, axis=1, kind="stable")
    ss = np.take_along_axis(sc, order, axis=1)
    margin2 = ss[:, 2] - ss[:, 1] if n_r >= 3 else np.full(T, np.inf)
    return dict(scores=sc, expert=order[:, 0].astype(np.int32), expert2=order[:, 1].astype(np.int32),
                margin2=margin2)


def qe_linear_top2(x: np.ndarray, x_is_bf16: bool, s: Optional[np.ndarray], qw: np.ndarray, s_w: np.ndarray,
                   a_bits: int, A_s, B_s, A_r, B_r, R, experts_override: Optional[np.ndarray] = None
                   ) -> Dict[str, np.ndarray]:
    """qe_linear with the two routed experts of route_top2, both corrections added.

    Reading (the pages give no rule for combining two experts): each routed expert is fitted
    to the error carried by its own cluster of token-dependent channels, so the two selected
    corrections are complementary and are summed with weight one.  experts_override [T, 2]
    replaces the router's pair (used only to re-evaluate near-tie tokens).
    """
    x32 = np.asarray(x, np.float32)
    xb = x32 if x_is_bf16 else bf16_round(x32)
    r2 = route_top2(xb, R)
    pair = np.stack([r2["expert"], r2["expert2"]], axis=1) if experts_override is None else \
        np.asarray(experts_override, np.int32)
    out = qe_linear(x, x_is_bf16, s, qw, s_w, a_bits, A_s=A_s, B_s=B_s, A_r=A_r, B_r=B_r, R=R,
                    expert_override=pair[:, 0])
    y = out["y64"] + routed_term(xb, A_r, B_r, pair[:, 1])
    out.update(r2)
    out["experts"] = pair
    out["y"] = y.astype(np.float32)
    out["y64"] = y
    return out


# ------------------------------------------------------------- channel top-k stat
def colmean_abs(W_f: np.ndarray) -> np.ndarray:
    """w = Mean_row(|W_f|): mean over output rows of |W_f|, one value per input channel.

    [DeepRead] "Method", first paragraph; [PaperDaily] "从观察到创新" (the row mean of
    the weight matrix gives each input channel's base importance).  Summed in
    float64, divided by d_out, rounded once to float32.
    """
    W = np.asarray(W_f, np.float64)
    return (np.abs(W).sum(axis=0) / W.shape[0]).astype(np.float32)


def channel_topk(x: np.ndarray, w: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """S_t = Top-k(|x_t| * w) per token, and the channel-frequency histogram.

    [DeepRead] "Method": per-token Top-k(|x_t| * w) gives the token's important
    channels; their selection frequency over the calibration tokens is then
    counted ([listing] Figure 3).  Scores are float32 products of |x| (at its
    stored precision) and w.  Order: score descending, channel index ascending.
    Returns topk int32 [T, k] and hist int64 [d_in].
    """
    x32 = np.asarray(x, np.float32)
    T, d = x32.shape
    sc = np.abs(x32) * np.asarray(w, np.float32)[None, :]
    j = np.broadcast_to(np.arange(d), sc.shape)
    order = np.lexsort((j, -sc), axis=-1)[:, :k].astype(np.int32)
    hist = np.bincount(order.reshape(-1), minlength=d).astype(np.int64)
    return order, hist


# ------------------------------------------------------------------ cost (Table 7)
def linear_cost(T: int, d_in: int, d_out: int, r_s: int, n_r: int, r_r: int) -> Dict[str, int]:
    """[listing] Table 7 generalised to d_in != d_out.

    Computation: T*d_in*d_out (quantized product) plus T*(d_in+d_out)*(r_s+r_r)
    (the shared expert and the one selected routed expert) plus T*d_in*N_r (router).
    Memory: d_in*d_out plus (d_in+d_out)*(r_s + N_r*r_r) adapter parameters.
    """
    return dict(
        int_macs=T * d_in * d_out,
        adapter_macs=T * (d_in + d_out) * (r_s + r_r) + T * d_in * n_r,
        weight_params=d_in * d_out,
        adapter_params=(d_in + d_out) * (r_s + n_r * r_r),
        router_params=d_in * n_r,
    )
