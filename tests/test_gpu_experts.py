"""GPU parity of the expert construction against the oracle: the quantization error, the
whitening weights, the rank-r subtraction, the randomized truncated SVD, the whole SE / RE
build, and the router's targets and ridge least-squares fit, at small sizes with ragged tiles
and at full layer sizes (sampled, or checked through properties that hold at any size)."""

import numpy as np
import pytest
import torch

from oracle import qe_expert_oracle as X

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def L():
    from quantized_linear_moe_amd import _libqe
    return _libqe


def _dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).to(DEV)


def _known(rng, d_in, d_out, sig):
    U, _ = np.linalg.qr(rng.standard_normal((d_in, len(sig))))
    V, _ = np.linalg.qr(rng.standard_normal((d_out, len(sig))))
    return U @ np.diag(sig) @ V.T


@pytest.mark.parametrize("w_bits,smooth,d_out,d_in", [(4, True, 96, 200), (3, True, 33, 4096), (4, False, 7, 1000),
                                                      (3, False, 64, 96)])
def test_quant_error_matches_oracle(L, w_bits, smooth, d_out, d_in):
    rng = np.random.default_rng(d_in + w_bits)
    W = (rng.standard_normal((d_out, d_in)) * 0.03).astype(np.float32)
    W[0, :5] = [0.2, -0.2, 0.0, 1e-9, -0.05]  # row with ties and tiny entries
    if d_out > 2:
        W[2] = 0.0  # an all-zero row
    s = rng.uniform(0.25, 4.0, d_in).astype(np.float32) if smooth else None
    E = torch.empty(d_out, d_in, device=DEV)
    L.qe_quant_error(_dev(W), _dev(s) if smooth else None, w_bits, E)
    torch.cuda.synchronize()
    ref = X.quant_error(W, s, w_bits)
    # same codes on both sides: a different code would move an entry by a whole step s_w / s
    scale = np.abs(W).max()
    assert np.max(np.abs(E.cpu().numpy() - ref)) <= 1e-6 * scale


def test_quant_error_full_size_sampled_rows(L):
    # Qwen2VL-72B down projection (29568 -> 8192), W4 with smoothing: rows sampled for the oracle
    rng = np.random.default_rng(11)
    d_out, d_in = 8192, 29568
    W = torch.randn(d_out, d_in, device=DEV) * 0.02
    s = torch.rand(d_in, device=DEV) * 1.5 + 0.5
    E = torch.empty_like(W)
    L.qe_quant_error(W, s, 4, E)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, d_out - 1], rng.choice(d_out, 14, replace=False)]))
    Wr = W[torch.as_tensor(rows, device=DEV)].cpu().numpy()
    ref = X.quant_error(Wr, s.cpu().numpy(), 4)
    got = E[torch.as_tensor(rows, device=DEV)].cpu().numpy()
    assert np.max(np.abs(got - ref)) <= 1e-6 * np.abs(Wr).max()


@pytest.mark.parametrize("dtype,T,d_in", [(torch.bfloat16, 1000, 300), (torch.float32, 256, 4096),
                                          (torch.bfloat16, 1, 17), (torch.float32, 4097, 64)])
def test_channel_rms_matches_oracle(L, dtype, T, d_in):
    rng = np.random.default_rng(T + d_in)
    x = torch.from_numpy((rng.standard_normal((T, d_in)) * rng.uniform(0.1, 10, d_in)).astype(np.float32)).to(dtype)
    x[:, 0] = 0.0  # a dead channel
    c = torch.empty(d_in, device=DEV)
    ws = torch.empty(L.qe_channel_rms_workspace_bytes(T, d_in), dtype=torch.uint8, device=DEV)
    L.qe_channel_rms(x.to(DEV), c, ws)
    torch.cuda.synchronize()
    ref = X.channel_rms(x.float().numpy())
    assert c[0].item() == 0.0
    assert np.allclose(c.cpu().numpy(), ref, rtol=2e-7, atol=0)


@pytest.mark.parametrize("d_out,d_in,r", [(100, 130, 5), (64, 64, 64), (257, 33, 1)])
def test_sub_lowrank_matches_definition(L, d_out, d_in, r):
    rng = np.random.default_rng(r)
    E = rng.standard_normal((d_out, d_in)).astype(np.float32)
    A = rng.standard_normal((d_in, r)).astype(np.float32)
    B = rng.standard_normal((r, d_out)).astype(np.float32)
    Ed = _dev(E)
    L.qe_sub_lowrank(Ed, _dev(A), _dev(B))
    torch.cuda.synchronize()
    ref = E.astype(np.float64) - (A.astype(np.float64) @ B.astype(np.float64)).T
    assert np.max(np.abs(Ed.cpu().numpy() - ref)) <= 1e-5 * np.sqrt(r) * 4


@pytest.mark.parametrize("d_out,d_in,k,rank,q,masked", [(300, 520, 20, 8, 2, False), (130, 1000, 40, 32, 1, True),
                                                       (200, 150, 100, 64, 2, False), (64, 64, 64, 64, 0, False)])
def test_lowrank_fit_matches_oracle(L, d_out, d_in, k, rank, q, masked):
    rng = np.random.default_rng(d_out * 3 + k)
    n_sig = min(d_in, d_out)
    sig = np.concatenate([np.linspace(10, 3, rank // 2 + 1), 0.3 * rng.uniform(0.5, 1, n_sig - rank // 2 - 1)])
    w = rng.uniform(0.2, 3.0, d_in)
    if masked:
        w[rng.random(d_in) < 0.6] = 0.0
    M = _known(rng, d_in, d_out, sig)
    with np.errstate(divide="ignore", invalid="ignore"):
        E = np.where(w[:, None] > 0, M / w[:, None], rng.standard_normal(M.shape)).T.astype(np.float32)
    omega = rng.standard_normal((d_out, k)).astype(np.float32)
    Ed, wd, od = _dev(E), _dev(w.astype(np.float32)), _dev(omega)
    ws = torch.empty(L.qe_lowrank_workspace_bytes(d_out, d_in, k), dtype=torch.uint8, device=DEV)
    A, B, s = L.qe_lowrank_fit(Ed, wd, od, rank, q, ws)
    Ar, Br, sr = X.randomized_lowrank(E, w.astype(np.float32), omega, rank, q)
    assert np.allclose(s, sr, rtol=2e-4, atol=1e-4 * sr[0])
    P, Pr = A.astype(np.float64) @ B, Ar @ Br
    wf = w.astype(np.float32).astype(np.float64)
    assert np.max(np.abs(wf[:, None] * (P - Pr))) <= 2e-4 * np.max(np.abs(wf[:, None] * Pr))
    assert np.all(A[w == 0] == 0)


def test_build_experts_matches_oracle(L):
    rng = np.random.default_rng(21)
    d_out, d_in, n_r, r_s, r_r, k, q = 128, 256, 4, 8, 4, 12, 3
    W = (rng.standard_normal((d_out, d_in)) * 0.04).astype(np.float32)
    s = rng.uniform(0.5, 2.0, d_in).astype(np.float32)
    x = (rng.standard_normal((500, d_in)) * rng.uniform(0.1, 5, d_in)).astype(np.float32)
    dep = rng.choice(d_in, 40, replace=False).astype(np.int32)
    labels = rng.integers(0, n_r, 40).astype(np.int32)
    labels[:2] = 3  # cluster 3 holds at least the first two
    om = rng.standard_normal((1 + n_r, d_out, k)).astype(np.float32)
    c = torch.empty(d_in, device=DEV)
    wsr = torch.empty(L.qe_channel_rms_workspace_bytes(500, d_in), dtype=torch.uint8, device=DEV)
    L.qe_channel_rms(_dev(x), c, wsr)
    ws = torch.empty(L.qe_build_experts_workspace_bytes(d_out, d_in, k, max(r_s, r_r)), dtype=torch.uint8, device=DEV)
    got = L.qe_build_experts(_dev(W), _dev(s), 4, c, dep, labels, n_r, r_s, r_r, _dev(om), q, ws)
    # the oracle computes its own whitening weights from the same calibration tokens
    ref = X.build_experts(W, s, 4, X.channel_rms(x), dep, labels, n_r, r_s, r_r, om, q)
    assert np.allclose(got["sigma_s"], ref["sigma_s"], rtol=5e-4)
    Ps, Psr = got["A_s"].astype(np.float64) @ got["B_s"], ref["A_s"] @ ref["B_s"]
    assert np.max(np.abs(Ps - Psr)) <= 5e-4 * np.max(np.abs(Psr))
    for g in range(n_r):
        ch = dep[labels == g]
        assert np.all(np.delete(got["A_r"][g], ch, axis=0) == 0)
        P, Pr = got["A_r"][g].astype(np.float64) @ got["B_r"][g], ref["A_r"][g] @ ref["B_r"][g]
        assert np.max(np.abs(P - Pr)) <= 2e-3 * max(np.max(np.abs(Pr)), 1e-30), g
        assert np.allclose(got["sigma_r"][g], ref["sigma_r"][g], rtol=2e-3, atol=1e-6 * ref["sigma_r"][g][0])


def test_build_experts_no_shared_no_routed(L):
    # r_shared = 0 (routed experts only, on E itself) and n_routed = 0 (shared expert only)
    rng = np.random.default_rng(22)
    d_out, d_in, k = 64, 96, 10
    W = (rng.standard_normal((d_out, d_in)) * 0.05).astype(np.float32)
    c = rng.uniform(0.5, 2, d_in).astype(np.float32)
    om = rng.standard_normal((3, d_out, k)).astype(np.float32)
    dep, labels = np.arange(20, dtype=np.int32), (np.arange(20) % 2).astype(np.int32)
    ws = torch.empty(L.qe_build_experts_workspace_bytes(d_out, d_in, k, 6), dtype=torch.uint8, device=DEV)
    got = L.qe_build_experts(_dev(W), None, 3, _dev(c), dep, labels, 2, 0, 6, _dev(om), 2, ws)
    ref = X.build_experts(W, None, 3, c, dep, labels, 2, 0, 6, om, 2)
    for g in range(2):
        P, Pr = got["A_r"][g].astype(np.float64) @ got["B_r"][g], ref["A_r"][g] @ ref["B_r"][g]
        assert np.max(np.abs(P - Pr)) <= 1e-3 * np.max(np.abs(Pr))
    got = L.qe_build_experts(_dev(W), None, 3, _dev(c), dep, labels, 0, 6, 0, _dev(om[:1]), 2, ws)
    ref = X.build_experts(W, None, 3, c, dep, labels, 0, 6, 0, om[:1], 2)
    P, Pr = got["A_s"].astype(np.float64) @ got["B_s"], ref["A_s"] @ ref["B_s"]
    assert np.max(np.abs(P - Pr)) <= 1e-3 * np.max(np.abs(Pr))


def test_lowrank_fit_full_size_properties(L):
    # Qwen2VL-72B down projection's quantization error (29568 -> 8192, W4, smoothing), rank 32,
    # k = 40, two power iterations.  At any size: diag(w) A = U_r S_r^(1/2) and B = S_r^(1/2) V_r^T
    # with orthonormal U_r, V_r, and the fit removes exactly sum(sigma^2) of |M|^2 (projection)
    d_out, d_in, k, r = 8192, 29568, 40, 32
    W = torch.randn(d_out, d_in, device=DEV) * 0.02
    s = torch.rand(d_in, device=DEV) * 1.5 + 0.5
    E = torch.empty_like(W)
    L.qe_quant_error(W, s, 4, E)
    del W
    w = torch.rand(d_in, device=DEV) * 3 + 0.1
    gen = torch.Generator(device=DEV).manual_seed(5)
    omega = torch.randn(d_out, k, device=DEV, generator=gen)
    ws = torch.empty(L.qe_lowrank_workspace_bytes(d_out, d_in, k), dtype=torch.uint8, device=DEV)
    A, B, sig = L.qe_lowrank_fit(E, w, omega, r, 2, ws)
    assert np.all(np.diff(sig) <= 0) and sig[-1] > 0
    wA = w.cpu().numpy().astype(np.float64)[:, None] * A
    assert np.allclose(wA.T @ wA, np.diag(sig), atol=2e-4 * sig[0])
    assert np.allclose(B.astype(np.float64) @ B.T.astype(np.float64), np.diag(sig), atol=2e-4 * sig[0])
    m2 = float(((E.double() * w.double()[None, :]) ** 2).sum())
    L.qe_sub_lowrank(E, torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV))
    r2 = float(((E.double() * w.double()[None, :]) ** 2).sum())
    assert abs((m2 - r2) - np.sum(sig ** 2)) <= 2e-3 * np.sum(sig ** 2)


def test_expert_argument_errors(L):
    E = torch.zeros(8, 16, device=DEV)
    om = torch.zeros(8, 4, device=DEV)
    ws = torch.empty(1 << 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(L.QEError):
        L.qe_lowrank_fit(E, None, om, 5, 1, ws)  # rank > k
    with pytest.raises(L.QEError):
        L.qe_lowrank_fit(E, None, torch.zeros(8, 9, device=DEV), 2, 1, ws)  # k > d_out
    with pytest.raises(L.QEError):
        L.qe_lowrank_fit(E, None, om, 2, 1, torch.empty(16, dtype=torch.uint8, device=DEV))  # workspace
    with pytest.raises(L.QEError):
        L.qe_quant_error(E, None, 5, E)
    c = torch.ones(16, device=DEV)
    with pytest.raises(L.QEError):  # a label outside [0, n_routed)
        L.qe_build_experts(E, None, 4, c, [1, 2], [0, 3], 2, 2, 2, torch.zeros(3, 8, 4, device=DEV), 1, ws)


@pytest.mark.parametrize("T,dtype", [(300, torch.bfloat16), (129, torch.float32), (1, torch.bfloat16)])
def test_router_targets_match_oracle(L, T, dtype):
    rng = np.random.default_rng(T)
    d_out, d_in, n_r, r_r = 96, 200, 3, 5
    E1 = (rng.standard_normal((d_out, d_in)) * 0.01).astype(np.float32)
    A = (rng.standard_normal((n_r, d_in, r_r)) * 0.1).astype(np.float32)
    A[1, 50:] = 0.0  # an expert on part of the channels
    B = (rng.standard_normal((n_r, r_r, d_out)) * 0.01).astype(np.float32)
    x = torch.from_numpy((rng.standard_normal((T, d_in)) * rng.uniform(0.2, 4, d_in)).astype(np.float32)).to(dtype)
    tg = torch.empty(T, n_r, device=DEV)
    ws = torch.empty(L.qe_router_targets_workspace_bytes(d_out, d_in, n_r, r_r), dtype=torch.uint8, device=DEV)
    L.qe_router_targets(_dev(E1), x.to(DEV), _dev(A), _dev(B), tg, ws)
    torch.cuda.synchronize()
    ref = X.router_targets(E1, x.float().numpy(), A, B)
    assert np.allclose(tg.cpu().numpy(), ref, rtol=2e-5, atol=1e-7 * np.max(ref))


def test_router_targets_full_size_sampled(L):
    # InternVL2-8B down projection (14336 -> 4096), W4 error, 8 experts of rank 32, 256 tokens;
    # the oracle recomputes 24 sampled tokens
    rng = np.random.default_rng(40)
    d_out, d_in, n_r, r_r, T = 4096, 14336, 8, 32, 256
    W = torch.randn(d_out, d_in, device=DEV) * 0.02
    E1 = torch.empty_like(W)
    L.qe_quant_error(W, None, 4, E1)
    del W
    A = torch.randn(n_r, d_in, r_r, device=DEV) * 0.01
    B = torch.randn(n_r, r_r, d_out, device=DEV) * 0.01
    x = (torch.randn(T, d_in, device=DEV) * 2).to(torch.bfloat16)
    tg = torch.empty(T, n_r, device=DEV)
    ws = torch.empty(L.qe_router_targets_workspace_bytes(d_out, d_in, n_r, r_r), dtype=torch.uint8, device=DEV)
    L.qe_router_targets(E1, x, A, B, tg, ws)
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 22, replace=False)]))
    ref = X.router_targets(E1.cpu().numpy(), x[torch.as_tensor(toks, device=DEV)].float().cpu().numpy(),
                           A.cpu().numpy(), B.cpu().numpy())
    assert np.allclose(tg.cpu().numpy()[toks], ref, rtol=1e-4)


@pytest.mark.parametrize("T,d_in,n_r,ridge,dtype", [(600, 128, 4, 1e-2, torch.float32), (100, 256, 8, 5e-2, torch.bfloat16),
                                                   (1000, 333, 1, 1e-3, torch.float32)])
def test_router_fit_matches_closed_form(L, T, d_in, n_r, ridge, dtype):
    rng = np.random.default_rng(T + d_in)
    x = torch.from_numpy((rng.standard_normal((T, d_in)) * rng.uniform(0.5, 2, d_in)).astype(np.float32)).to(dtype)
    tgt = rng.uniform(0.0, 1.0, (T, n_r)).astype(np.float32)
    ws = torch.empty(L.qe_router_fit_workspace_bytes(T, d_in, n_r), dtype=torch.uint8, device=DEV)
    R, it = L.qe_router_fit(x.to(DEV), _dev(tgt), ridge, 2000, 1e-7, ws)
    ref = X.router_fit(x.float().numpy(), tgt, ridge)
    assert it < 2000
    assert np.max(np.abs(R - ref)) <= 2e-3 * np.max(np.abs(ref))
