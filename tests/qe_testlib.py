"""Helpers shared by the GPU parity tests: build a prepared QE linear on the device
from the seeded generators, evaluate the oracle on the same inputs, and compare
with the benchmark spec's tolerances (codes/accumulators/routes/top-k bit-exact except
router near-ties; float outputs within max|dy| / max|y_ref| <= 2e-3)."""

import os
from typing import Dict, Optional

import numpy as np
import torch

from oracle import qe_oracle as O

Y_TOL = 2e-3          # max |y_gpu - y_ref| / max |y_ref|
NEAR_TIE_REL = 1e-4   # router scores closer than this (relative) may pick either expert


def f32(t) -> Optional[np.ndarray]:
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.astype(np.float32)
    return t.float().cpu().numpy()


def oracle_for(params: Dict[str, object], x: torch.Tensor, w_bits: int, a_bits: int,
               tokens: Optional[np.ndarray] = None, qw_sw=None) -> Dict[str, np.ndarray]:
    """Oracle output of one QE linear on (a subset of) the tokens of x."""
    xs = x if tokens is None else x[torch.as_tensor(tokens)]
    qw, s_w = qw_sw if qw_sw is not None else O.quant_weights(params["W_f"], params["s"] if a_bits != 16 else None, w_bits)
    out = O.qe_linear(f32(xs), xs.dtype == torch.bfloat16, params["s"] if a_bits != 16 else None, qw, s_w, a_bits,
                      A_s=f32(params.get("A_s")), B_s=f32(params.get("B_s")), A_r=f32(params.get("A_r")),
                      B_r=f32(params.get("B_r")), R=f32(params.get("R")))
    out["qw"], out["s_w"] = qw, s_w
    return out


def near_ties(ref: Dict[str, np.ndarray]) -> np.ndarray:
    if "margin" not in ref:
        return np.zeros(0, bool)
    return ref["margin"] < NEAR_TIE_REL * ref["margin_scale"]


def check_routing(ref: Dict[str, np.ndarray], gpu_expert: np.ndarray) -> np.ndarray:
    """Bit-exact routes except near-ties; near-tie tokens must pick one of the two smallest scores.
    Returns the mask of tokens whose GPU route differs from the oracle's (all near-ties)."""
    e_ref = ref["expert"]
    near = near_ties(ref)
    diff = gpu_expert != e_ref
    report_routing(os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0], ref, gpu_expert)
    assert not np.any(diff & ~near), f"{int(np.sum(diff & ~near))} routing mismatches away from near-ties"
    if np.any(diff):
        order = np.argsort(ref["scores"][diff], axis=1, kind="stable")[:, :2]
        assert np.all((order == gpu_expert[diff][:, None]).any(axis=1))
    return diff


def rel_err(y: np.ndarray, y_ref: np.ndarray) -> float:
    denom = float(np.max(np.abs(y_ref)))
    return float(np.max(np.abs(y.astype(np.float64) - y_ref.astype(np.float64)))) / max(denom, 1e-30)


def check_y(y_gpu: np.ndarray, ref: Dict[str, np.ndarray], params, x_sub: torch.Tensor, w_bits: int, a_bits: int,
            gpu_expert: Optional[np.ndarray] = None, tol: float = Y_TOL) -> float:
    y_ref = ref["y64"].copy()
    if gpu_expert is not None and "expert" in ref:
        diff = check_routing(ref, gpu_expert)
        if np.any(diff):  # re-evaluate near-tie tokens with the GPU's (equally valid) expert
            idx = np.nonzero(diff)[0]
            qw, s_w = ref["qw"], ref["s_w"]
            alt = O.qe_linear(f32(x_sub[torch.as_tensor(idx)]), x_sub.dtype == torch.bfloat16,
                              params["s"] if a_bits != 16 else None, qw, s_w, a_bits,
                              A_s=f32(params.get("A_s")), B_s=f32(params.get("B_s")), A_r=f32(params.get("A_r")),
                              B_r=f32(params.get("B_r")), R=f32(params.get("R")), expert_override=gpu_expert[idx])
            y_ref[idx] = alt["y64"]
    err = rel_err(y_gpu, y_ref)
    assert err <= tol, f"max|dy|/max|y_ref| = {err:.3e} > {tol}"
    return err


# Routing reports: every GPU parity test that compares routes records the near-tie count
# and the number of differing routes here; tests/conftest.py prints them at the end of the
# run (also under -q), so the counts are kept in the test log.
ROUTING_REPORT = []


def report_routing(label: str, ref: Dict[str, np.ndarray], gpu_expert: np.ndarray) -> None:
    near = near_ties(ref)
    diff = gpu_expert != ref["expert"]
    n = len(gpu_expert)
    hist = np.bincount(gpu_expert, minlength=ref["scores"].shape[1]).tolist()
    ROUTING_REPORT.append(f"{label}: tokens {n}, near-ties {int(near.sum())}, differing routes {int(diff.sum())}, "
                          f"GPU expert histogram {hist}")
    # the synthetic workloads keep near-ties rare; a flood of them would hide routing bugs
    assert int(near.sum()) <= max(3, n // 200), f"{label}: {int(near.sum())} near-tie tokens of {n}"
