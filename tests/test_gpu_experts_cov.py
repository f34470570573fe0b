"""GPU expert construction by covariance whitening against the exact oracle.

The oracle (oracle/qe_expert_oracle.py: error_cov_lowrank, build_experts_cov) is the exact
minimizer of sum_t |(E - A_hat) x_t|^2 (eigenvectors of the error-output covariance), with
no randomness.  The GPU runs the randomized subspace iteration on the same operator, so it
approaches the minimizer: products A B within a stated tolerance where the spectrum has a
gap, and at the InternVL2-8B down size (14336 -> 4096, 4096 calibration tokens, rank 32,
k = 40 columns, 2 power iterations) a residual within 1 % of the Eckart-Young optimum.

Why 1 %: the residual of any rank-r fit is rho^2 = |Z|^2 - captured, and the optimum
captures the top-r energy exactly, so rho / rho* - 1 <= deficit / (2 rho*^2), where deficit
is the top-r energy the randomized basis misses.  With k = r + 8 columns and 2 power
iterations the missed part of each direction decays as (sigma_{k+1} / sigma_j)^(4q+2)
(Halko, Martinsson and Tropp, Section 10.4); on this workload the residual energy rho*^2 is
several times the top-r energy, so even a deficit of a few percent of the captured energy
stays far below 1 % of rho*.  The test prints the measured excess.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import qe_expert_oracle as X

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def L():
    from quantized_linear_moe_amd import _libqe
    return _libqe


def _dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).to(DEV)


def _planted(rng, d_out, d_in, T, r_true):
    """E with a decaying spectrum plus noise, and correlated calibration tokens."""
    U, _ = np.linalg.qr(rng.standard_normal((d_out, r_true)))
    V, _ = np.linalg.qr(rng.standard_normal((d_in, r_true)))
    sig = 2.0 ** -np.arange(r_true, dtype=np.float64) * 0.5 + 0.05
    E = (U * sig) @ V.T + 1e-3 * rng.standard_normal((d_out, d_in))
    F = rng.standard_normal((T, d_in // 4))
    Xc = F @ rng.standard_normal((d_in // 4, d_in)) / np.sqrt(d_in // 4) + 0.3 * rng.standard_normal((T, d_in))
    Xc *= rng.uniform(0.3, 3.0, d_in)[None, :]
    return E.astype(np.float32), Xc.astype(np.float32)


@pytest.mark.parametrize("d_out,d_in,T,rank,k", [(256, 640, 512, 16, 24), (200, 96, 300, 8, 16), (97, 333, 130, 5, 9)])
def test_lowrank_fit_cov_matches_exact(L, d_out, d_in, T, rank, k):
    # E of exact rank `rank` (plus 1e-5 noise): the operator Z = E X^T has a gap of four
    # orders of magnitude after `rank`, so the randomized fit must reproduce the exact one
    rng = np.random.default_rng(d_out + d_in)
    U, _ = np.linalg.qr(rng.standard_normal((d_out, rank)))
    V, _ = np.linalg.qr(rng.standard_normal((d_in, rank)))
    E = ((U * np.geomspace(1.0, 0.05, rank)) @ V.T + 1e-5 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    _, Xc = _planted(rng, d_out, d_in, T, rank)
    omega = rng.standard_normal((T, k)).astype(np.float32)
    ws = torch.empty(L.qe_lowrank_cov_workspace_bytes(d_out, d_in, T, k), dtype=torch.uint8, device=DEV)
    A, B, sig = L.qe_lowrank_fit_cov(_dev(E), _dev(Xc), None, _dev(omega), rank, 2, ws)
    Ar, Br, sr = X.error_cov_lowrank(E, Xc, rank)
    assert np.allclose(sig, sr, rtol=1e-3), (sig, sr)
    P, Pr = A.astype(np.float64) @ B, Ar @ Br
    assert np.max(np.abs(P - Pr)) <= 2e-3 * np.max(np.abs(Pr))
    res, opt = X.output_residual(E, Xc, A, B), X.output_residual(E, Xc, Ar, Br)
    zn = np.linalg.norm(Xc.astype(np.float64) @ E.T.astype(np.float64))
    assert res <= opt * 1.01 + 1e-5 * zn, (res, opt, zn)


@pytest.mark.parametrize("d_out,d_in,T,rank,k", [(256, 640, 512, 16, 24), (97, 333, 130, 5, 9)])
def test_lowrank_fit_cov_flat_tail_residual_bound(L, d_out, d_in, T, rank, k):
    # a decaying head and a flat tail: the leading directions (large gaps) are found exactly,
    # the ones inside the flat tail only approximately, and the residual stays within 1 % of
    # the Eckart-Young optimum
    rng = np.random.default_rng(d_out + d_in + 1)
    E, Xc = _planted(rng, d_out, d_in, T, 2 * rank)
    omega = rng.standard_normal((T, k)).astype(np.float32)
    ws = torch.empty(L.qe_lowrank_cov_workspace_bytes(d_out, d_in, T, k), dtype=torch.uint8, device=DEV)
    A, B, sig = L.qe_lowrank_fit_cov(_dev(E), _dev(Xc), None, _dev(omega), rank, 2, ws)
    Ar, Br, sr = X.error_cov_lowrank(E, Xc, rank)
    assert np.allclose(sig[:3], sr[:3], rtol=1e-4), (sig[:3], sr[:3])
    assert np.all(sig <= sr * (1 + 1e-5))  # a projection never captures more than the optimum
    res, opt = X.output_residual(E, Xc, A, B), X.output_residual(E, Xc, Ar, Br)
    print(f"residual {res:.6e} vs optimum {opt:.6e}: excess {res / opt - 1:.2e}")
    assert res <= opt * 1.01, (res, opt)


def test_lowrank_fit_cov_narrow_mask_is_exact(L):
    # a cluster of 20 channels and rank 24: the fit reproduces E on the cluster's columns
    rng = np.random.default_rng(5)
    d_out, d_in, T, k = 160, 512, 256, 32
    E = rng.standard_normal((d_out, d_in)).astype(np.float32)
    Xc = (rng.standard_normal((T, d_in)) * rng.uniform(0.5, 2, d_in)).astype(np.float32)
    ch = np.sort(rng.choice(d_in, 20, replace=False))
    mask = np.zeros(d_in, np.float32)
    mask[ch] = 1
    omega = rng.standard_normal((T, k)).astype(np.float32)
    ws = torch.empty(L.qe_lowrank_cov_workspace_bytes(d_out, d_in, T, k), dtype=torch.uint8, device=DEV)
    A, B, sig = L.qe_lowrank_fit_cov(_dev(E), _dev(Xc), _dev(mask), _dev(omega), 24, 2, ws)
    assert np.all(A[mask == 0] == 0)
    assert np.all(sig[20:] == 0) and np.all(sig[:20] > 0)
    rec = (A[ch].astype(np.float64) @ B).T
    assert np.max(np.abs(rec - E[:, ch])) <= 1e-4 * np.max(np.abs(E[:, ch]))


def test_build_experts_cov_matches_oracle(L):
    rng = np.random.default_rng(31)
    d_out, d_in, T, n_r, r_s, r_r, k = 192, 384, 600, 4, 8, 8, 16
    W = (rng.standard_normal((d_out, d_in)) * 0.04).astype(np.float32)
    s = rng.uniform(0.5, 2.0, d_in).astype(np.float32)
    _, Xc = _planted(rng, d_out, d_in, T, 8)
    Xc[:, 7] *= 25  # an outlier channel: the whitening must follow it
    xb = torch.from_numpy(Xc).to(torch.bfloat16)
    xf = xb.float().numpy()  # the adapters read bf16(x): the oracle takes the same values
    dep = rng.choice(d_in, 48, replace=False).astype(np.int32)
    labels = (np.arange(48) % n_r).astype(np.int32)
    om = rng.standard_normal((1 + n_r, T, k)).astype(np.float32)
    ws = torch.empty(L.qe_build_experts_cov_workspace_bytes(d_out, d_in, T, k, max(r_s, r_r)), dtype=torch.uint8,
                     device=DEV)
    got = L.qe_build_experts_cov(_dev(W), _dev(s), 4, xb.to(DEV), dep, labels, n_r, r_s, r_r, _dev(om), 2, ws)
    ref = X.build_experts_cov(W, s, 4, xf, dep, labels, n_r, r_s, r_r)
    E = X.quant_error(W, s, 4)
    rs, rs_opt = X.output_residual(E, xf, got["A_s"], got["B_s"]), X.output_residual(E, xf, ref["A_s"], ref["B_s"])
    assert rs <= rs_opt * (1 + 1e-2), (rs, rs_opt)
    # each RE fits the residual the GPU's own SE leaves (E_1 = E - (A_s B_s)^T)
    E1 = E - (got["A_s"].astype(np.float64) @ got["B_s"]).T
    for g in range(n_r):  # 12 channels per cluster, rank 8
        ch = np.sort(dep[labels == g])
        assert np.all(np.delete(got["A_r"][g], ch, axis=0) == 0)
        E1g = E1[:, ch]
        Ag, Bg, _ = X.error_cov_lowrank(E1g, xf[:, ch], r_r)
        r_gpu = X.output_residual(E1g, xf[:, ch], got["A_r"][g][ch], got["B_r"][g])
        r_opt = X.output_residual(E1g, xf[:, ch], Ag, Bg)
        assert r_gpu <= r_opt * (1 + 2e-2) + 1e-6 * np.linalg.norm(xf[:, ch] @ E1g.T), (g, r_gpu, r_opt)


def test_build_experts_cov_internvl2_8b_down_vs_exact(L):
    # InternVL2-8B down projection: 14336 -> 4096, W4 with smoothing, the synthetic down input
    # (4096 tokens), rank 32 shared and 8 routed experts of rank 32 on 8 clusters of 32
    # token-dependent channels, k = 40 columns, 2 power iterations
    cfg = synth.get_config("internvl2_8b")
    spec = next(l for l in cfg.linears if l.name == "down")
    params = synth.gen_linear(cfg, spec)
    W, s = params["W_f"], params["s"]
    x = synth.gen_activations(cfg, spec.stream)  # bf16 [4096, 14336]
    xf = x.float().numpy()
    T, d_in, d_out, k, r, n_r = xf.shape[0], spec.d_in, spec.d_out, 40, 32, 8
    rng = np.random.default_rng(41)
    dep = rng.choice(d_in, n_r * 32, replace=False).astype(np.int32)
    labels = (np.arange(n_r * 32) % n_r).astype(np.int32)
    om = torch.randn(1 + n_r, T, k, device=DEV, generator=torch.Generator(device=DEV).manual_seed(3))
    ws = torch.empty(L.qe_build_experts_cov_workspace_bytes(d_out, d_in, T, k, r), dtype=torch.uint8, device=DEV)
    got = L.qe_build_experts_cov(_dev(W), _dev(s), 4, x.to(DEV), dep, labels, n_r, r, r, om, 2, ws)
    del ws
    E = X.quant_error(W, s, 4)
    As, Bs, ss = X.error_cov_lowrank(E, xf, r)
    Z = xf.astype(np.float64) @ E.T  # [T, d_out]
    total = float(np.sum(Z * Z))
    opt = float(np.sqrt(max(total - np.sum(ss ** 2), 0.0)))
    res = float(np.linalg.norm(Z - (xf.astype(np.float64) @ got["A_s"]) @ got["B_s"]))
    # the diagonal whitening's exact fit, for comparison
    Ad, Bd, _ = X.whitened_lowrank(E, X.channel_rms(xf), r)
    res_diag = float(np.linalg.norm(Z - (xf.astype(np.float64) @ Ad) @ Bd))
    print(f"SE residual {res:.6e}, optimum {opt:.6e} (excess {res / opt - 1:.2e}), diagonal whitening "
          f"{res_diag:.6e}; top sigma GPU {got['sigma_s'][:3]}, exact {ss[:3]}")
    assert res <= opt * 1.01
    assert res < res_diag
    assert np.allclose(got["sigma_s"][:4], ss[:4], rtol=1e-3)
    # routed experts: each on its cluster's residual columns, against the exact fit
    E1 = E - (got["A_s"].astype(np.float64) @ got["B_s"]).T
    for g in range(n_r):
        ch = np.sort(dep[labels == g])
        assert np.all(np.delete(got["A_r"][g], ch, axis=0) == 0)
        Ag, Bg, _ = X.error_cov_lowrank(E1[:, ch], xf[:, ch], r)
        r_opt = X.output_residual(E1[:, ch], xf[:, ch], Ag, Bg)
        r_gpu = X.output_residual(E1[:, ch], xf[:, ch], got["A_r"][g][ch], got["B_r"][g])
        scale = np.linalg.norm(xf[:, ch] @ E1[:, ch].T)
        assert r_gpu <= r_opt * 1.01 + 1e-5 * scale, (g, r_gpu, r_opt, scale)
