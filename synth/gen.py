"""Seeded tensor generators.

Every tensor has its own random stream, keyed by (config seed, tensor name), so
adding a tensor never shifts another.  numpy's PCG64 generator is used for all
draws.  Storage dtypes: activations are bf16 (or fp32 where the workload says
so), the full-precision weight W_f and the smoothing vector are fp32, and the
adapters and the router are bf16.  Conversion to bf16 is torch's
round-to-nearest-even storage cast of the drawn fp32 values.
"""

import zlib
from typing import Dict, Optional

import numpy as np
import torch

from .configs import ActRecipe, LinearSpec, QEConfig

WEIGHT_STD = 0.02  # W_f, A, B, R ~ N(0, 0.02)


def rng_for(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng([int(seed), zlib.crc32(name.encode("utf-8"))])


def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _distinct_rows(rng: np.random.Generator, n_rows: int, n_pick: int, pool: np.ndarray) -> np.ndarray:
    """n_rows independent draws of n_pick distinct entries of `pool`."""
    if n_pick == 0:
        return np.zeros((n_rows, 0), dtype=np.int64)
    idx = rng.integers(0, len(pool), size=(n_rows, n_pick))
    while True:
        s = np.sort(idx, axis=1)
        bad = np.nonzero((s[:, 1:] == s[:, :-1]).any(axis=1))[0]
        if len(bad) == 0:
            break
        idx[bad] = rng.integers(0, len(pool), size=(len(bad), n_pick))
    return pool[idx]


def gen_activations(cfg: QEConfig, stream: str, T: Optional[int] = None) -> torch.Tensor:
    """Activation tensor [T, d] of one stream, in its storage dtype (CPU).

    Gaussian tokens; per modality a fixed set of channels is scaled on every
    token and each token scales a few extra channels drawn from the modality's
    pool.  Returns torch.bfloat16 or torch.float32.
    """
    recipe: ActRecipe = cfg.acts[stream]
    d = cfg.stream_dim(stream)
    rng = rng_for(cfg.seed, "act/" + stream)
    n_tok_total = sum(m[0] for m in recipe.modalities)
    x = _normal(rng, (n_tok_total, d))

    # channel sets: fixed sets and pools of the modalities are disjoint
    perm = rng.permutation(d)
    cursor = 0
    row0 = 0
    for mi, (n_tok, n_fixed, f_mult, pool_n, n_tok_pick, t_mult) in enumerate(recipe.modalities):
        if recipe.fixed_channels is not None and mi == 0:
            fixed = np.asarray(recipe.fixed_channels, dtype=np.int64)
            perm = np.array([c for c in perm if c not in set(fixed.tolist())], dtype=np.int64)
        else:
            fixed = perm[cursor:cursor + n_fixed]
            cursor += n_fixed
        if pool_n > 0:
            pool = perm[cursor:cursor + pool_n]
            cursor += pool_n
        else:
            pool = perm[cursor:]
        xr = x[row0:row0 + n_tok]  # view into x
        xr[:, fixed] *= np.float32(f_mult)
        picks = _distinct_rows(rng, n_tok, n_tok_pick, pool)
        r_idx = np.repeat(np.arange(n_tok), n_tok_pick)
        xr[r_idx, picks.reshape(-1)] *= np.float32(t_mult)
        row0 += n_tok

    if T is not None:
        x = x[:T] if T <= x.shape[0] else np.concatenate([x] * (-(-T // x.shape[0])))[:T]
    t = torch.from_numpy(np.ascontiguousarray(x))
    if recipe.dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16)


def gen_linear(cfg: QEConfig, lin: LinearSpec, with_weight: bool = True) -> Dict[str, object]:
    """All parameters of one QE linear (CPU tensors / arrays).

    W_f   float32 ndarray [d_out, d_in]   full-precision weight, N(0, 0.02)
    s     float32 ndarray [d_in] or None smoothing vector, U(0.5, 2); None for A16
    A_s   bf16 [d_in, r_s],  B_s bf16 [r_s, d_out]          shared expert
    A_r   bf16 [N_r, d_in, r_r], B_r bf16 [N_r, r_r, d_out]  routed experts
    R     bf16 [d_in, N_r]                                   router
    """
    key = f"{cfg.name}/{lin.name}"
    out: Dict[str, object] = {}
    if with_weight:
        out["W_f"] = _normal(rng_for(cfg.seed, key + "/W_f"), (lin.d_out, lin.d_in), WEIGHT_STD)
    if cfg.a_bits == 16:
        out["s"] = None
    else:
        out["s"] = rng_for(cfg.seed, key + "/s").uniform(0.5, 2.0, size=lin.d_in).astype(np.float32)
    out["A_s"] = _bf16(_normal(rng_for(cfg.seed, key + "/A_s"), (lin.d_in, cfg.r_shared), WEIGHT_STD))
    out["B_s"] = _bf16(_normal(rng_for(cfg.seed, key + "/B_s"), (cfg.r_shared, lin.d_out), WEIGHT_STD))
    out["A_r"] = _bf16(_normal(rng_for(cfg.seed, key + "/A_r"), (cfg.n_routed, lin.d_in, cfg.r_routed), WEIGHT_STD))
    out["B_r"] = _bf16(_normal(rng_for(cfg.seed, key + "/B_r"), (cfg.n_routed, cfg.r_routed, lin.d_out), WEIGHT_STD))
    out["R"] = _bf16(_normal(rng_for(cfg.seed, key + "/R"), (lin.d_in, cfg.n_routed), WEIGHT_STD))
    return out
