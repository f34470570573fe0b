"""Device-side holder of one prepared QE linear (memory management + marshalling only).

torch allocates the device buffers; libqe packs, lays out and computes.
"""

from typing import Dict, Optional

import numpy as np
import torch

from . import _libqe as L


def _dev(a, device, dtype=None):
    if a is None:
        return None
    t = a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.contiguous().to(device)


class QELinear:
    """One QE linear: packed weights, smoothing, shared/routed adapters and router, prepared for libqe."""

    def __init__(self, d_in: int, d_out: int, w_bits: int, a_bits: int, r_shared: int, n_routed: int,
                 r_routed: int, device="cuda"):
        self.device = torch.device(device)
        self.lin = L.make_linear(d_in, d_out, w_bits, a_bits, r_shared, n_routed, r_routed if n_routed else 0)
        nbytes = L.qe_prepared_bytes(self.lin)
        if nbytes == 0:
            raise ValueError("unsupported QE linear configuration")
        self.prep = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.lin.prep = self.prep.data_ptr()
        self.packed = None
        self.w_scale = None

    @classmethod
    def from_params(cls, params: Dict[str, object], w_bits: int, a_bits: int, device="cuda",
                    packed: Optional[np.ndarray] = None, w_scale: Optional[np.ndarray] = None) -> "QELinear":
        """params: W_f (float32 [d_out, d_in]) or (packed, w_scale); s; A_s, B_s, A_r, B_r, R (bf16)."""
        A_s, B_s, A_r, B_r, R = (params.get(k) for k in ("A_s", "B_s", "A_r", "B_r", "R"))
        s = params.get("s") if a_bits != 16 else None  # weight-only layers carry no smoothing
        if packed is None:
            W_f = params["W_f"]
            d_out, d_in = W_f.shape
            packed, w_scale = L.qe_pack_weights(W_f, s, w_bits)
        else:
            d_out, d_in = params["d_out"], params["d_in"]
        r_s = 0 if A_s is None else A_s.shape[1]
        n_r = 0 if A_r is None else A_r.shape[0]
        r_r = 0 if A_r is None else A_r.shape[2]
        self = cls(d_in, d_out, w_bits, a_bits, r_s, n_r, r_r, device)
        dev = self.device
        bufs = dict(
            w_packed=_dev(packed, dev), w_scale=_dev(w_scale, dev), smooth=_dev(s, dev, torch.float32),
            A_s=_dev(A_s, dev, torch.bfloat16) if r_s else None, B_s=_dev(B_s, dev, torch.bfloat16) if r_s else None,
            A_r=_dev(A_r, dev, torch.bfloat16) if n_r else None, B_r=_dev(B_r, dev, torch.bfloat16) if n_r else None,
            R=_dev(R, dev, torch.bfloat16) if n_r else None,
        )
        L.qe_prepare(self.lin, bufs["w_packed"], bufs["w_scale"], bufs["smooth"], bufs["A_s"], bufs["B_s"],
                     bufs["A_r"], bufs["B_r"], bufs["R"], self.prep)
        torch.cuda.current_stream(dev).synchronize()  # inputs may be freed after the prepare work
        self.packed, self.w_scale = packed, w_scale
        return self

    def workspace(self, T: int) -> torch.Tensor:
        return torch.empty(max(L.qe_workspace_bytes(self.lin, T), 256), dtype=torch.uint8, device=self.device)

    def forward(self, x: torch.Tensor, y: Optional[torch.Tensor] = None, expert_out: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None) -> torch.Tensor:
        T = x.shape[0]
        if y is None:
            dt = torch.bfloat16 if self.lin.y_dtype == L.QE_BF16 else torch.float32
            y = torch.empty(T, self.lin.d_out, dtype=dt, device=self.device)
        if ws is None:
            ws = self.workspace(T)
        L.qe_linear_forward(self.lin, x, y, expert_out, ws)
        return y
