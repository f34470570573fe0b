"""ctypes binding of libqe (include/qe.h).  Argument marshalling only.

Every function here has the name of the C entry point it wraps, takes torch
tensors (device memory) or numpy arrays (host memory) where the C function takes
pointers, passes torch's current HIP stream, and raises QEError on a non-zero
status.  No computation of the hot path happens in Python: if the shared library
is missing, importing this module fails.
"""

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqe.so")

QE_OK, QE_ERR_INVALID_ARG, QE_ERR_UNSUPPORTED, QE_ERR_ALIGNMENT, QE_ERR_WORKSPACE, QE_ERR_HIP = range(6)
QE_F32, QE_BF16 = 0, 1


class QEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {_lib.qe_status_string(status).decode()}"
        if status == QE_ERR_HIP:
            msg += f" (hipError {_lib.qe_last_hip_error()})"
        super().__init__(msg)


class qe_linear(ctypes.Structure):
    _fields_ = [
        ("d_in", ctypes.c_int32),
        ("d_out", ctypes.c_int32),
        ("w_bits", ctypes.c_int32),
        ("a_bits", ctypes.c_int32),
        ("r_shared", ctypes.c_int32),
        ("n_routed", ctypes.c_int32),
        ("r_routed", ctypes.c_int32),
        ("y_dtype", ctypes.c_int32),
        ("prep", ctypes.c_void_p),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libqe.so not found at {LIB_PATH}; build it with `python quantized_linear_moe_amd/build.py` "
            "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.POINTER(ctypes.c_double)
    LP = ctypes.POINTER(qe_linear)
    sig = {
        "qe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "qe_last_hip_error": (ctypes.c_int, []),
        "qe_version": (ctypes.c_char_p, []),
        "qe_pack_weights": (ctypes.c_int, [P, P, I, I, I, P, P]),
        "qe_prepared_bytes": (Z, [LP]),
        "qe_prepare": (ctypes.c_int, [LP, P, P, P, P, P, P, P, P, P, P]),
        "qe_workspace_bytes": (Z, [LP, I]),
        "qe_quant_act": (ctypes.c_int, [P, I, P, I, I, I, P, P, P]),
        "qe_route": (ctypes.c_int, [LP, P, I, I, P, P, P, P, P, P, Z, P]),
        "qe_adapter_inputs": (ctypes.c_int, [LP, P, I, I, P, P, P, P, Z, P]),
        "qe_wq_gemm": (ctypes.c_int, [LP, P, P, P, I, I, P, P, P, P, P, P, P, Z, P]),
        "qe_routed_lora": (ctypes.c_int, [LP, P, I, I, P, P, P, P, P, Z, P]),
        "qe_linear_prologue": (ctypes.c_int, [LP, P, I, I, P, P, P, P, P, P, P, Z, P]),
        "qe_linear_forward": (ctypes.c_int, [LP, P, I, I, P, P, P, Z, P]),
        "qe_group_prologue": (ctypes.c_int, [P, I, P, I, I, P, P, P, P, P, P, P, P, P]),
        "qe_group_forward": (ctypes.c_int, [P, I, P, I, I, P, P, P, P, P]),
        "qe_group_gemm": (ctypes.c_int, [P, I, P, P, I, P, P, P, P, P, P, P, P]),
        "qe_noalloc_scratch_bytes": (Z, []),
        "qe_linear_forward_noalloc": (ctypes.c_int, [LP, P, I, I, P, P, P]),
        "qe_colmean_abs": (ctypes.c_int, [P, I, I, I, P, P]),
        "qe_channel_topk": (ctypes.c_int, [P, I, P, I, I, I, P, P, P]),
        "qe_partition_channels": (ctypes.c_int, [P, I, I, I, P, P, P]),
        "qe_cooccur_workspace_bytes": (Z, [I, I]),
        "qe_cooccur": (ctypes.c_int, [P, I, I, P, I, I, P, P, Z, P]),
        "qe_cluster_channels": (ctypes.c_int, [P, I, ctypes.c_int64, I, ctypes.c_double, P, P, P, P]),
        "qe_linear_cost": (ctypes.c_int, [LP, I, I, I, D, D, D]),
        "qe_top2_workspace_bytes": (Z, [LP, I]),
        "qe_linear_forward_top2": (ctypes.c_int, [LP, P, I, I, P, P, P, P, Z, P]),
        "qe_quant_error": (ctypes.c_int, [P, P, I, I, I, P, P]),
        "qe_channel_rms_workspace_bytes": (Z, [I, I]),
        "qe_channel_rms": (ctypes.c_int, [P, I, I, I, P, P, Z, P]),
        "qe_sub_lowrank": (ctypes.c_int, [P, I, I, P, P, I, P]),
        "qe_lowrank_workspace_bytes": (Z, [I, I, I]),
        "qe_lowrank_fit": (ctypes.c_int, [P, I, I, P, P, I, I, I, P, P, P, P, Z, P]),
        "qe_build_experts_workspace_bytes": (Z, [I, I, I, I]),
        "qe_build_experts": (ctypes.c_int, [P, P, I, I, I, P, P, P, I, I, I, I, P, I, I, P, P, P, P, P, P, P, Z, P]),
        "qe_lowrank_cov_workspace_bytes": (Z, [I, I, I, I]),
        "qe_lowrank_fit_cov": (ctypes.c_int, [P, I, I, P, I, P, P, I, I, I, P, P, P, P, Z, P]),
        "qe_build_experts_cov_workspace_bytes": (Z, [I, I, I, I, I]),
        "qe_build_experts_cov": (ctypes.c_int, [P, P, I, I, I, P, I, I, P, P, I, I, I, I, P, I, I, P, P, P, P, P, P,
                                                P, Z, P]),
        "qe_router_targets_workspace_bytes": (Z, [I, I, I, I]),
        "qe_router_targets": (ctypes.c_int, [P, I, I, P, I, I, P, P, I, I, P, P, Z, P]),
        "qe_router_fit_workspace_bytes": (Z, [I, I, I]),
        "qe_router_fit": (ctypes.c_int, [P, I, I, I, P, I, ctypes.c_double, I, ctypes.c_double, P, P, P, Z, P]),
        "qe_probe_mfma_i8": (ctypes.c_int, [P, I, I, I, D, P]),
        "qe_probe_mfma_bf16": (ctypes.c_int, [P, I, I, I, D, P]),
        "qe_probe_copy": (ctypes.c_int, [P, P, Z, P]),
        "qe_probe_read_sink_bytes": (Z, []),
        "qe_probe_read": (ctypes.c_int, [P, Z, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()
EXPORTED = (
    "qe_status_string", "qe_last_hip_error", "qe_version", "qe_pack_weights", "qe_prepared_bytes", "qe_prepare",
    "qe_workspace_bytes", "qe_quant_act", "qe_route", "qe_adapter_inputs", "qe_wq_gemm", "qe_routed_lora",
    "qe_linear_prologue", "qe_linear_forward", "qe_noalloc_scratch_bytes", "qe_linear_forward_noalloc",
    "qe_group_prologue", "qe_group_forward", "qe_group_gemm", "qe_colmean_abs", "qe_channel_topk", "qe_linear_cost",
    "qe_probe_mfma_i8", "qe_probe_mfma_bf16", "qe_probe_copy", "qe_probe_read_sink_bytes", "qe_probe_read", "qe_partition_channels", "qe_cooccur_workspace_bytes",
    "qe_cooccur", "qe_cluster_channels", "qe_top2_workspace_bytes", "qe_linear_forward_top2", "qe_quant_error", "qe_channel_rms_workspace_bytes", "qe_channel_rms",
    "qe_sub_lowrank", "qe_lowrank_workspace_bytes", "qe_lowrank_fit", "qe_build_experts_workspace_bytes",
    "qe_build_experts", "qe_lowrank_cov_workspace_bytes", "qe_lowrank_fit_cov",
    "qe_build_experts_cov_workspace_bytes", "qe_build_experts_cov", "qe_router_targets_workspace_bytes", "qe_router_targets", "qe_router_fit_workspace_bytes",
    "qe_router_fit",
)


# ----------------------------------------------------------------- marshalling
def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return QE_BF16
    if t.dtype == torch.float32:
        return QE_F32
    raise TypeError(f"activations must be bf16 or float32, got {t.dtype}")


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(st: int, where: str):
    if st != QE_OK:
        raise QEError(st, where)


def make_linear(d_in, d_out, w_bits, a_bits, r_shared, n_routed, r_routed, prep=None) -> qe_linear:
    return qe_linear(d_in, d_out, w_bits, a_bits, r_shared, n_routed, r_routed, 0, _ptr(prep))


def qe_status_string(status: int) -> str:
    return _lib.qe_status_string(status).decode()


def qe_last_hip_error() -> int:
    return _lib.qe_last_hip_error()


def qe_version() -> str:
    return _lib.qe_version().decode()


def qe_pack_weights(W_f: np.ndarray, s: Optional[np.ndarray], w_bits: int):
    """Host quantize + pack; returns (packed bytes as uint8 ndarray, w_scale float32 ndarray)."""
    W_f = np.ascontiguousarray(W_f, dtype=np.float32)
    d_out, d_in = W_f.shape
    s_arr = None if s is None else np.ascontiguousarray(s, dtype=np.float32)
    nbytes = d_out * d_in // 2 if w_bits == 4 else d_out * d_in * 3 // 8
    packed = np.empty(nbytes, dtype=np.uint8)
    w_scale = np.empty(d_out, dtype=np.float32)
    _check(_lib.qe_pack_weights(_ptr(W_f), _ptr(s_arr), d_out, d_in, w_bits, _ptr(packed), _ptr(w_scale)),
           "qe_pack_weights")
    return packed, w_scale


def qe_prepared_bytes(lin: qe_linear) -> int:
    return _lib.qe_prepared_bytes(ctypes.byref(lin))


def qe_prepare(lin: qe_linear, w_packed, w_scale, smooth, A_s, B_s, A_r, B_r, R, prep, stream=None):
    _check(_lib.qe_prepare(ctypes.byref(lin), _ptr(w_packed), _ptr(w_scale), _ptr(smooth), _ptr(A_s), _ptr(B_s),
                           _ptr(A_r), _ptr(B_r), _ptr(R), _ptr(prep), _stream(stream)), "qe_prepare")


def qe_workspace_bytes(lin: qe_linear, T: int) -> int:
    return _lib.qe_workspace_bytes(ctypes.byref(lin), T)


def qe_quant_act(x, smooth, a_bits, codes, s_x, stream=None):
    T, d_in = x.shape
    _check(_lib.qe_quant_act(_ptr(x), _dtype_code(x), _ptr(smooth), T, d_in, a_bits, _ptr(codes), _ptr(s_x),
                             _stream(stream)), "qe_quant_act")


def qe_route(lin, x, scores, expert, counts, offsets, perm, ws, stream=None):
    _check(_lib.qe_route(ctypes.byref(lin), _ptr(x), _dtype_code(x), x.shape[0], _ptr(scores), _ptr(expert),
                         _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(ws), ws.numel() * ws.element_size(),
                         _stream(stream)), "qe_route")


def qe_adapter_inputs(lin, x, expert, u, v, ws, stream=None):
    _check(_lib.qe_adapter_inputs(ctypes.byref(lin), _ptr(x), _dtype_code(x), x.shape[0], _ptr(expert), _ptr(u),
                                  _ptr(v), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "qe_adapter_inputs")


def qe_wq_gemm(lin, codes, s_x, x, T, u, v, expert, y, acc_debug, ws, stream=None, perm=None):
    xd = _dtype_code(x) if x is not None else QE_BF16
    _check(_lib.qe_wq_gemm(ctypes.byref(lin), _ptr(codes), _ptr(s_x), _ptr(x), xd, T, _ptr(u), _ptr(v), _ptr(expert),
                           _ptr(perm), _ptr(y), _ptr(acc_debug), _ptr(ws), ws.numel() * ws.element_size(),
                           _stream(stream)), "qe_wq_gemm")


def qe_routed_lora(lin, x, expert, offsets, perm, y, ws, stream=None):
    _check(_lib.qe_routed_lora(ctypes.byref(lin), _ptr(x), _dtype_code(x), x.shape[0], _ptr(expert), _ptr(offsets),
                               _ptr(perm), _ptr(y), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "qe_routed_lora")


def qe_linear_prologue(lin, x, codes, s_x, u, v, expert, ws, stream=None, perm=None):
    _check(_lib.qe_linear_prologue(ctypes.byref(lin), _ptr(x), _dtype_code(x), x.shape[0], _ptr(codes), _ptr(s_x),
                                   _ptr(u), _ptr(v), _ptr(expert), _ptr(perm), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)), "qe_linear_prologue")


def rank_pad(r: int) -> int:
    """Row stride (elements) of the adapter-input buffers u / v for rank r."""
    return 0 if r <= 0 else (r + 31) // 32 * 32


def qe_linear_forward(lin, x, y, expert_out, ws, stream=None):
    _check(_lib.qe_linear_forward(ctypes.byref(lin), _ptr(x), _dtype_code(x), x.shape[0], _ptr(y), _ptr(expert_out),
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "qe_linear_forward")


def _ptr_array(items):
    return (ctypes.c_void_p * len(items))(*[_ptr(t) for t in items])


def _lin_array(lins):
    return (ctypes.POINTER(qe_linear) * len(lins))(*[ctypes.pointer(l) for l in lins])


def qe_group_prologue(lins, x, codes, s_x, u, v, expert, ws, perm=None, stream=None):
    """Prologues of linears that read the same x (lists, one entry per linear; see include/qe.h)."""
    n = len(lins)
    perm = perm if perm is not None else [None] * n
    wsb = (ctypes.c_size_t * n)(*[w.numel() * w.element_size() for w in ws])
    _check(_lib.qe_group_prologue(_lin_array(lins), n, _ptr(x), _dtype_code(x), x.shape[0], _ptr_array(codes),
                                  _ptr_array(s_x), _ptr_array(u), _ptr_array(v), _ptr_array(expert),
                                  _ptr_array(perm), _ptr_array(ws), wsb, _stream(stream)), "qe_group_prologue")


def qe_group_forward(lins, x, ys, expert_out, ws, stream=None):
    """QE linears that read the same x (lists, one entry per linear; expert_out a list or None)."""
    n = len(lins)
    eo = _ptr_array(expert_out) if expert_out is not None else None
    wsb = (ctypes.c_size_t * n)(*[w.numel() * w.element_size() for w in ws])
    _check(_lib.qe_group_forward(_lin_array(lins), n, _ptr(x), _dtype_code(x), x.shape[0], _ptr_array(ys), eo,
                                 _ptr_array(ws), wsb, _stream(stream)), "qe_group_forward")


def qe_group_gemm(lins, codes, s_x, T, u, v, expert, ys, ws, perm=None, stream=None):
    """Main products of linears that read the same input (lists, one entry per linear)."""
    n = len(lins)
    perm = perm if perm is not None else [None] * n
    wsb = (ctypes.c_size_t * n)(*[w.numel() * w.element_size() for w in ws])
    _check(_lib.qe_group_gemm(_lin_array(lins), n, _ptr_array(codes), _ptr_array(s_x), T, _ptr_array(u),
                              _ptr_array(v), _ptr_array(expert), _ptr_array(perm), _ptr_array(ys), _ptr_array(ws), wsb,
                              _stream(stream)), "qe_group_gemm")


def qe_noalloc_scratch_bytes() -> int:
    return _lib.qe_noalloc_scratch_bytes()


def qe_linear_forward_noalloc(lin, x, y, expert_out, stream=None):
    """qe_linear_forward with the library's per-GPU scratch array as its workspace."""
    _check(_lib.qe_linear_forward_noalloc(ctypes.byref(lin), _ptr(x), _dtype_code(x), x.shape[0], _ptr(y),
                                          _ptr(expert_out), _stream(stream)), "qe_linear_forward_noalloc")


def qe_colmean_abs(W, w, stream=None):
    d_out, d_in = W.shape
    _check(_lib.qe_colmean_abs(_ptr(W), _dtype_code(W), d_out, d_in, _ptr(w), _stream(stream)), "qe_colmean_abs")


def qe_channel_topk(x, w, k, topk, hist, stream=None):
    T, d_in = x.shape
    _check(_lib.qe_channel_topk(_ptr(x), _dtype_code(x), _ptr(w), T, d_in, k, _ptr(topk), _ptr(hist),
                                _stream(stream)), "qe_channel_topk")


def qe_partition_channels(hist: np.ndarray, k: int, n_r: int):
    """Host frequency partition; returns (indep int32 [k], dep int32 [n_r*k], slot int32 [d_in])."""
    hist = np.ascontiguousarray(hist, dtype=np.uint32)
    d_in = hist.shape[0]
    indep = np.empty(max(k, 0), np.int32)
    dep = np.empty(max(k * n_r, 0), np.int32)
    slot = np.empty(d_in, np.int32)
    _check(_lib.qe_partition_channels(_ptr(hist), d_in, k, n_r, _ptr(indep), _ptr(dep), _ptr(slot)),
           "qe_partition_channels")
    return indep, dep, slot


def qe_cooccur_workspace_bytes(T, n_dep) -> int:
    return _lib.qe_cooccur_workspace_bytes(T, n_dep)


def qe_cooccur(topk, slot, n_dep, cooc, ws, stream=None):
    """Enqueue cooc += O^T O for the token-dependent channels (device tensors; ws: a byte
    tensor of at least qe_cooccur_workspace_bytes(T, n_dep) bytes)."""
    T, k = topk.shape
    _check(_lib.qe_cooccur(_ptr(topk), T, k, _ptr(slot), slot.shape[0], n_dep, _ptr(cooc), _ptr(ws),
                           ws.numel() * ws.element_size(), _stream(stream)), "qe_cooccur")


def qe_cluster_channels(cooc: np.ndarray, T: int, n_clusters: int, threshold: float = 0.2, outputs: bool = False):
    """Host NPMI similarity, spectral embedding and K-Means; returns labels int32 [n_dep], and with
    outputs=True also (similarity, eigvals, embedding)."""
    cooc = np.ascontiguousarray(cooc, dtype=np.uint32)
    n = cooc.shape[0]
    labels = np.empty(n, np.int32)
    sim = np.empty((n, n), np.float64) if outputs else None
    ev = np.empty(max(n_clusters, 0), np.float64) if outputs else None
    emb = np.empty((n, max(n_clusters, 0)), np.float64) if outputs else None
    _check(_lib.qe_cluster_channels(_ptr(cooc), n, T, n_clusters, threshold, _ptr(labels), _ptr(sim), _ptr(ev),
                                    _ptr(emb)), "qe_cluster_channels")
    return (labels, sim, ev, emb) if outputs else labels


def qe_top2_workspace_bytes(lin: qe_linear, T: int) -> int:
    return _lib.qe_top2_workspace_bytes(ctypes.byref(lin), T)


def qe_linear_forward_top2(lin: qe_linear, x, y, expert_out=None, expert2_out=None, ws=None, stream=None):
    """Enqueue the QE linear with the two routed experts of smallest score per token."""
    T = x.shape[0]
    _check(_lib.qe_linear_forward_top2(ctypes.byref(lin), _ptr(x), _dtype_code(x), T, _ptr(y), _ptr(expert_out),
                                       _ptr(expert2_out), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                       _stream(stream)), "qe_linear_forward_top2")


def qe_quant_error(W_f, s, w_bits, E, stream=None):
    """Enqueue E = W_f - W_q (device float32 tensors; s may be None)."""
    d_out, d_in = W_f.shape
    _check(_lib.qe_quant_error(_ptr(W_f), _ptr(s), d_out, d_in, w_bits, _ptr(E), _stream(stream)), "qe_quant_error")


def qe_channel_rms(x, c, ws, stream=None):
    """Enqueue c = per-channel RMS of x over its tokens (ws: a device byte tensor of at least
    qe_channel_rms_workspace_bytes(T, d_in) bytes)."""
    T, d_in = x.shape
    _check(_lib.qe_channel_rms(_ptr(x), _dtype_code(x), T, d_in, _ptr(c), _ptr(ws), ws.numel() * ws.element_size(),
                               _stream(stream)), "qe_channel_rms")


def qe_channel_rms_workspace_bytes(T: int, d_in: int) -> int:
    return _lib.qe_channel_rms_workspace_bytes(T, d_in)


def qe_sub_lowrank(E, A, B, stream=None):
    """Enqueue E -= (A B)^T in place (device float32: E [d_out, d_in], A [d_in, r], B [r, d_out])."""
    d_out, d_in = E.shape
    _check(_lib.qe_sub_lowrank(_ptr(E), d_out, d_in, _ptr(A), _ptr(B), A.shape[1], _stream(stream)), "qe_sub_lowrank")


def qe_lowrank_workspace_bytes(d_out: int, d_in: int, k: int) -> int:
    return _lib.qe_lowrank_workspace_bytes(d_out, d_in, k)


def qe_lowrank_fit(E, w, omega, rank, power_iters, ws, stream=None):
    """Randomized truncated SVD of diag(w) E^T (device inputs; omega [d_out, k]); returns host
    numpy (A [d_in, rank] float32, B [rank, d_out] float32, sigma [rank] float64)."""
    d_out, d_in = E.shape
    k = omega.shape[1]
    A = np.empty((d_in, rank), np.float32)
    B = np.empty((rank, d_out), np.float32)
    sig = np.empty(rank, np.float64)
    _check(_lib.qe_lowrank_fit(_ptr(E), d_out, d_in, _ptr(w), _ptr(omega), k, rank, power_iters, _ptr(A), _ptr(B),
                               _ptr(sig), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "qe_lowrank_fit")
    return A, B, sig


def qe_build_experts_workspace_bytes(d_out: int, d_in: int, k: int, r_max: int) -> int:
    return _lib.qe_build_experts_workspace_bytes(d_out, d_in, k, r_max)


def qe_build_experts(W_f, s, w_bits, c, dep_channels, labels, n_routed, r_shared, r_routed, omegas, power_iters, ws,
                     stream=None):
    """SE and REs of one linear (device W_f, s, c, omegas [1 + n_routed, d_out, k]; host dep_channels
    and labels); returns a dict of host numpy arrays A_s, B_s, A_r, B_r (float32), sigma_s, sigma_r."""
    d_out, d_in = W_f.shape
    k = omegas.shape[2]
    dep = np.ascontiguousarray(dep_channels, dtype=np.int32)
    lab = np.ascontiguousarray(labels, dtype=np.int32)
    rr = r_routed if n_routed else 0
    out = dict(A_s=np.empty((d_in, r_shared), np.float32), B_s=np.empty((r_shared, d_out), np.float32),
               A_r=np.empty((n_routed, d_in, rr), np.float32), B_r=np.empty((n_routed, rr, d_out), np.float32),
               sigma_s=np.empty(r_shared, np.float64), sigma_r=np.empty((n_routed, rr), np.float64))
    _check(_lib.qe_build_experts(_ptr(W_f), _ptr(s), d_out, d_in, w_bits, _ptr(c), _ptr(dep), _ptr(lab), dep.shape[0],
                                 n_routed, r_shared, r_routed, _ptr(omegas), k, power_iters, _ptr(out["A_s"]),
                                 _ptr(out["B_s"]), _ptr(out["A_r"]), _ptr(out["B_r"]), _ptr(out["sigma_s"]),
                                 _ptr(out["sigma_r"]), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "qe_build_experts")
    return out


def qe_lowrank_cov_workspace_bytes(d_out: int, d_in: int, T: int, k: int) -> int:
    return _lib.qe_lowrank_cov_workspace_bytes(d_out, d_in, T, k)


def qe_lowrank_fit_cov(E, X, mask, omega, rank, power_iters, ws, stream=None):
    """Covariance-whitened fit of E diag(mask) on tokens X (device float32 [T, d_in]; omega [T, k]);
    returns host numpy (A [d_in, rank] float32, B [rank, d_out] float32, sigma [rank] float64)."""
    d_out, d_in = E.shape
    T, k = omega.shape
    A = np.empty((d_in, rank), np.float32)
    B = np.empty((rank, d_out), np.float32)
    sig = np.empty(rank, np.float64)
    _check(_lib.qe_lowrank_fit_cov(_ptr(E), d_out, d_in, _ptr(X), T, _ptr(mask), _ptr(omega), k, rank, power_iters,
                                   _ptr(A), _ptr(B), _ptr(sig), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)), "qe_lowrank_fit_cov")
    return A, B, sig


def qe_build_experts_cov_workspace_bytes(d_out: int, d_in: int, T: int, k: int, r_max: int) -> int:
    return _lib.qe_build_experts_cov_workspace_bytes(d_out, d_in, T, k, r_max)


def qe_build_experts_cov(W_f, s, w_bits, x, dep_channels, labels, n_routed, r_shared, r_routed, omegas, power_iters,
                         ws, stream=None):
    """SE and REs by covariance whitening over the calibration tokens x (device W_f, s, x [T, d_in],
    omegas [1 + n_routed, T, k]; host dep_channels and labels); returns a dict of host numpy arrays
    A_s, B_s, A_r, B_r (float32), sigma_s, sigma_r."""
    d_out, d_in = W_f.shape
    T = x.shape[0]
    k = omegas.shape[2]
    dep = np.ascontiguousarray(dep_channels, dtype=np.int32)
    lab = np.ascontiguousarray(labels, dtype=np.int32)
    rr = r_routed if n_routed else 0
    out = dict(A_s=np.empty((d_in, r_shared), np.float32), B_s=np.empty((r_shared, d_out), np.float32),
               A_r=np.empty((n_routed, d_in, rr), np.float32), B_r=np.empty((n_routed, rr, d_out), np.float32),
               sigma_s=np.empty(r_shared, np.float64), sigma_r=np.empty((n_routed, rr), np.float64))
    _check(_lib.qe_build_experts_cov(_ptr(W_f), _ptr(s), d_out, d_in, w_bits, _ptr(x), _dtype_code(x), T, _ptr(dep),
                                     _ptr(lab), dep.shape[0], n_routed, r_shared, r_routed, _ptr(omegas), k,
                                     power_iters, _ptr(out["A_s"]), _ptr(out["B_s"]), _ptr(out["A_r"]),
                                     _ptr(out["B_r"]), _ptr(out["sigma_s"]), _ptr(out["sigma_r"]), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)), "qe_build_experts_cov")
    return out


def qe_router_targets_workspace_bytes(d_out: int, d_in: int, n_routed: int, r_routed: int) -> int:
    return _lib.qe_router_targets_workspace_bytes(d_out, d_in, n_routed, r_routed)


def qe_router_targets(E1, x, A_r, B_r, target, ws, stream=None):
    """Enqueue target[t, g] = mean_i |x_t (E1^T - A_g B_g)|_i (device tensors; A_r, B_r float32)."""
    d_out, d_in = E1.shape
    n_r, _, r_r = A_r.shape
    _check(_lib.qe_router_targets(_ptr(E1), d_out, d_in, _ptr(x), _dtype_code(x), x.shape[0], _ptr(A_r), _ptr(B_r),
                                  n_r, r_r, _ptr(target), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "qe_router_targets")


def qe_router_fit_workspace_bytes(T: int, d_in: int, n_routed: int) -> int:
    return _lib.qe_router_fit_workspace_bytes(T, d_in, n_routed)


def qe_router_fit(x, target, ridge, max_iters, tol, ws, stream=None):
    """Ridge least-squares router fit by conjugate gradients; returns (R host float32 [d_in, n_r], iterations)."""
    T, d_in = x.shape
    n_r = target.shape[1]
    R = np.empty((d_in, n_r), np.float32)
    it = ctypes.c_int32()
    _check(_lib.qe_router_fit(_ptr(x), _dtype_code(x), T, d_in, _ptr(target), n_r, ridge, max_iters, tol, _ptr(R),
                              ctypes.byref(it), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "qe_router_fit")
    return R, it.value


def qe_probe_mfma_i8(out, blocks, iters, operands=0, stream=None):
    """Enqueue the int8 MFMA throughput probe; returns the integer operations enqueued."""
    ops = ctypes.c_double()
    _check(_lib.qe_probe_mfma_i8(_ptr(out), blocks, iters, operands, ctypes.byref(ops), _stream(stream)),
           "qe_probe_mfma_i8")
    return ops.value


def qe_probe_mfma_bf16(out, blocks, iters, operands=0, stream=None):
    """Enqueue the bf16 MFMA throughput probe; returns the floating-point operations enqueued."""
    flops = ctypes.c_double()
    _check(_lib.qe_probe_mfma_bf16(_ptr(out), blocks, iters, operands, ctypes.byref(flops), _stream(stream)),
           "qe_probe_mfma_bf16")
    return flops.value


def qe_probe_copy(src, dst, nbytes, stream=None):
    """Enqueue the streaming copy probe of nbytes from src to dst (traffic: 2 * nbytes)."""
    _check(_lib.qe_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)), "qe_probe_copy")


def qe_probe_read_sink_bytes() -> int:
    return _lib.qe_probe_read_sink_bytes()


def qe_probe_read(src, nbytes, sink, stream=None):
    _check(_lib.qe_probe_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)), "qe_probe_read")


def qe_linear_cost(lin, T, n_distinct, x_bytes):
    a, b, c = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _check(_lib.qe_linear_cost(ctypes.byref(lin), T, n_distinct, x_bytes, ctypes.byref(a), ctypes.byref(b),
                               ctypes.byref(c)), "qe_linear_cost")
    return a.value, b.value, c.value


def raw_library():
    """The ctypes CDLL handle (for tests that call entry points with raw pointers)."""
    return _lib
