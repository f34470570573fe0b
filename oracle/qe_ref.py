"""ctypes front of the plain C oracle (oracle/qe_ref.c) of the QE linear hot path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the library.  `build()` compiles the C file with gcc
(-O3, x86-64-v3, OpenMP, no floating-point contraction) into oracle/libqe_ref.so; the
functions below marshal numpy arrays and return numpy arrays.  Semantics and citations
are in the C file.
"""

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qe_ref.c")
LIB = os.path.join(HERE, "libqe_ref.so")
# x86-64-v3 (AVX2) rather than -march=native: the library is built once and may run on
# another host CPU than the one that compiled it.
CFLAGS = ["-O3", "-march=x86-64-v3", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC",
          "-shared", "-Wall"]


def build() -> str:
    tmp = LIB + ".tmp"
    r = subprocess.run(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed for the C oracle:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise ImportError(f"{LIB} is not built; run __graft_entry__.build() (gcc) first")
        L = ctypes.CDLL(LIB)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.qo_num_threads.restype = I
        L.qo_set_threads.argtypes = [I]
        L.qo_quant_act.argtypes = [P, P, I64, I64, I, P, P]
        L.qo_quant_weights.argtypes = [P, P, I64, I64, I, P, P]
        L.qo_main_acc.argtypes = [P, P, I64, I64, I64, P]
        L.qo_route.argtypes = [P, P, I64, I64, I, P, P, P, P, P, P, P]
        L.qo_qe_linear.argtypes = [P, I, P, P, P, I64, I64, I64, I, I, P, P, I, I, P, P, P, P, P, P, P, P, P, P, P]
        L.qo_channel_topk.argtypes = [P, P, I64, I64, I, P, P]
        L.qo_colmean_abs.argtypes = [P, I64, I64, P]
        _lib = L
    return _lib


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    return None if a is None else a.ctypes.data


def num_threads() -> int:
    return lib().qo_num_threads()


def set_threads(n: int) -> None:
    lib().qo_set_threads(int(n))


def quant_act(x, s, a_bits):
    x = _c(x, np.float32)
    s = _c(s, np.float32)
    T, d = x.shape
    codes = np.empty((T, d), np.int8)
    s_x = np.empty(T, np.float32)
    assert lib().qo_quant_act(_p(x), _p(s), T, d, a_bits, _p(codes), _p(s_x)) == 0
    return codes, s_x


def quant_weights(W, s, w_bits):
    W = _c(W, np.float32)
    s = _c(s, np.float32)
    d_out, d_in = W.shape
    codes = np.empty((d_out, d_in), np.int8)
    s_w = np.empty(d_out, np.float32)
    assert lib().qo_quant_weights(_p(W), _p(s), d_out, d_in, w_bits, _p(codes), _p(s_w)) == 0
    return codes, s_w


def main_acc(qx, qw):
    qx, qw = _c(qx, np.int8), _c(qw, np.int8)
    T, d_in = qx.shape
    d_out = qw.shape[0]
    acc = np.empty((T, d_out), np.int32)
    if lib().qo_main_acc(_p(qx), _p(qw), T, d_in, d_out, _p(acc)) != 0:
        raise OverflowError("an accumulator leaves the int32 range")
    return acc


def route(xb, R):
    xb, R = _c(xb, np.float32), _c(R, np.float32)
    T, d_in = xb.shape
    n_r = R.shape[1]
    sc = np.empty((T, n_r), np.float64)
    e = np.empty(T, np.int32)
    mg, ms = np.empty(T), np.empty(T)
    counts, offsets, perm = np.empty(n_r, np.int32), np.empty(n_r + 1, np.int32), np.empty(T, np.int32)
    assert lib().qo_route(_p(xb), _p(R), T, d_in, n_r, _p(sc), _p(e), _p(mg), _p(ms), _p(counts), _p(offsets),
                          _p(perm)) == 0
    return dict(scores=sc, expert=e, margin=mg, margin_scale=ms, counts=counts, offsets=offsets, perm=perm)


def qe_linear(x, x_is_bf16: bool, s, qw, s_w, a_bits: int, A_s=None, B_s=None, A_r=None, B_r=None, R=None,
              expert_override: Optional[np.ndarray] = None, want_acc: bool = False) -> Dict[str, np.ndarray]:
    """The whole QE linear (see qo_qe_linear in the C file).  Returns y (float32), y64,
    and expert / margin / margin_scale / codes / s_x / acc where they apply."""
    x = _c(x, np.float32)
    qw = _c(qw, np.int8)
    s_w = _c(s_w, np.float32)
    s = _c(s, np.float32) if a_bits != 16 else None
    T, d_in = x.shape
    d_out = qw.shape[0]
    r_s = 0 if A_s is None else A_s.shape[1]
    n_r = 0 if R is None else R.shape[1]
    r_r = 0 if A_r is None else A_r.shape[2]
    A_s, B_s, A_r, B_r, R = (_c(a, np.float32) for a in (A_s, B_s, A_r, B_r, R))
    ov = _c(expert_override, np.int32)
    y = np.empty((T, d_out), np.float64)
    out: Dict[str, np.ndarray] = {}
    e = mg = ms = codes = s_x = acc = None
    if n_r > 0:
        e, mg, ms = np.empty(T, np.int32), np.empty(T), np.empty(T)
    if a_bits != 16:
        codes, s_x = np.empty((T, d_in), np.int8), np.empty(T, np.float32)
        if want_acc:
            acc = np.empty((T, d_out), np.int32)
    st = lib().qo_qe_linear(_p(x), int(bool(x_is_bf16)), _p(s), _p(qw), _p(s_w), T, d_in, d_out, a_bits, r_s,
                            _p(A_s), _p(B_s), n_r, r_r, _p(A_r), _p(B_r), _p(R), _p(ov), _p(y), _p(e), _p(mg),
                            _p(ms), _p(codes), _p(s_x), _p(acc))
    if st < 0:
        raise ValueError("unsupported bit width")
    if st == 1:
        raise OverflowError("an accumulator leaves the int32 range")
    if n_r > 0:
        out.update(expert=e, margin=mg, margin_scale=ms)
    if a_bits != 16:
        out.update(codes=codes, s_x=s_x)
        if want_acc:
            out["acc"] = acc
    out["y64"] = y
    out["y"] = y.astype(np.float32)
    return out


def channel_topk(x, w, k):
    x, w = _c(x, np.float32), _c(w, np.float32)
    T, d = x.shape
    topk = np.empty((T, k), np.int32)
    hist = np.empty(d, np.int64)
    assert lib().qo_channel_topk(_p(x), _p(w), T, d, k, _p(topk), _p(hist)) == 0
    return topk, hist


def colmean_abs(W):
    W = _c(W, np.float32)
    d_out, d_in = W.shape
    w = np.empty(d_in, np.float32)
    lib().qo_colmean_abs(_p(W), d_out, d_in, _p(w))
    return w
