"""Pins of the expert-construction oracle (CPU): hand-worked quantization errors, matrices of
known singular values, the whitening objective on activations with a known covariance, and
the structure the SE / RE construction must have."""

import numpy as np
import pytest

from oracle import qe_expert_oracle as X
from oracle import qe_expert_oracle as X_


def _orth(rng, n, m):
    q, _ = np.linalg.qr(rng.standard_normal((n, m)))
    return q


def _known_svd(rng, d_in, d_out, sig):
    """M = U diag(sig) V^T with random orthonormal U [d_in, n], V [d_out, n]."""
    n = len(sig)
    U, V = _orth(rng, d_in, n), _orth(rng, d_out, n)
    return U, np.asarray(sig, dtype=np.float64), V, U @ np.diag(sig) @ V.T


def test_quant_error_hand_example():
    # W4, one row [1, 0.4, -0.3, 0] (float32): s_w = fl(1/7); codes rint(w / s_w) = 7, 3, -2, 0;
    # E = w - s_w * code, worked out in exact decimals of the float32 values
    W = np.array([[1.0, 0.4, -0.3, 0.0]], dtype=np.float32)
    E = X.quant_error(W, None, 4)
    want = [-4.4703483581542969e-08, -0.0285714417695999146, -0.0142857134342193604, 0.0]
    assert np.allclose(E[0], want, rtol=0, atol=1e-15)


def test_quant_error_with_smoothing_hand_example():
    # s = [2, 0.5, 1, 1] maps the row [0.5, 0.8, -0.3, 0] onto the row above (same codes and
    # s_w); W_q = s_w * code / s, so E = [0.5 - 7 s_w / 2, 0.8 - 3 s_w / 0.5, -0.3 + 2 s_w, 0]
    W = np.array([[0.5, 0.8, -0.3, 0.0]], dtype=np.float32)
    s = np.array([2.0, 0.5, 1.0, 1.0], dtype=np.float32)
    E = X.quant_error(W, s, 4)
    want = [-2.2351741790771484e-08, -0.0571428835391998291, -0.0142857134342193604, 0.0]
    assert np.allclose(E[0], want, rtol=0, atol=1e-15)


@pytest.mark.parametrize("w_bits", [3, 4])
def test_quant_error_zero_on_the_grid(w_bits):
    # weights that are exactly code * 2^-5 / s (s powers of two), each row reaching the top
    # code, quantize without error
    rng = np.random.default_rng(1)
    qmax = 7 if w_bits == 4 else 3
    q = rng.integers(-qmax, qmax + 1, size=(6, 32))
    q[:, 0] = qmax
    s = 2.0 ** rng.integers(-2, 3, size=32)
    W = (q * 2.0 ** -5 / s[None, :]).astype(np.float32)
    assert np.array_equal(X.quant_error(W, s.astype(np.float32), w_bits), np.zeros((6, 32)))
    assert np.array_equal(X.quant_error(W * s[None, :].astype(np.float32), None, w_bits), np.zeros((6, 32)))


def test_channel_rms_hand_example():
    c = X.channel_rms(np.array([[3.0, 0.0], [4.0, 1.0]]))
    assert np.allclose(c, [np.sqrt(12.5), np.sqrt(0.5)], rtol=0, atol=1e-15)


def test_whitened_lowrank_recovers_known_singular_values():
    rng = np.random.default_rng(2)
    U, sig, V, M = _known_svd(rng, 12, 9, [9, 7, 5, 3, 2, 1, 0.5, 0.2, 0.1])
    w = rng.uniform(0.5, 2.0, 12)
    E = (M / w[:, None]).T  # so that diag(w) E^T = M
    A, B, s = X.whitened_lowrank(E, w, 3)
    assert np.allclose(s, sig[:3], rtol=1e-12)
    assert np.allclose(w[:, None] * (A @ B), U[:, :3] @ np.diag(sig[:3]) @ V[:, :3].T, atol=1e-12)
    # Eckart-Young: the residual is the energy of the dropped singular values
    res = np.linalg.norm(M - w[:, None] * (A @ B))
    assert abs(res - np.sqrt(np.sum(sig[3:] ** 2))) < 1e-12


def test_whitening_minimizes_the_output_error():
    # activations with orthogonal columns of RMS w (rows of a Hadamard matrix): the expected
    # output error sum_t |x_t (E^T - A B)|^2 is T |diag(w)(E^T - A B)|^2, so the whitened fit
    # beats the unwhitened one and random perturbations of its factors
    rng = np.random.default_rng(3)
    H = np.array([[1.0]])
    for _ in range(4):
        H = np.block([[H, H], [H, -H]])
    T, d_in, d_out, r = 16, 10, 7, 2
    w = rng.uniform(0.1, 3.0, d_in)
    Xc = H[:, :d_in] * w[None, :]
    assert np.allclose(X.channel_rms(Xc), w)
    E = rng.standard_normal((d_out, d_in))
    obj = lambda A, B: np.sum((Xc @ (E.T - A @ B)) ** 2)
    A, B, _ = X.whitened_lowrank(E, w, r)
    best = obj(A, B)
    A1, B1, _ = X.whitened_lowrank(E, np.ones(d_in), r)
    assert obj(A1, B1) > best * (1 + 1e-6)
    for _ in range(20):
        assert obj(A + 1e-3 * rng.standard_normal(A.shape), B + 1e-3 * rng.standard_normal(B.shape)) > best


def test_zero_weights_restrict_the_fit():
    # channels with weight 0 get zero rows in A, and the fit equals the fit of the submatrix
    rng = np.random.default_rng(4)
    E = rng.standard_normal((8, 11))
    w = rng.uniform(0.5, 1.5, 11)
    keep = np.array([0, 2, 3, 7, 9])
    wm = np.zeros(11)
    wm[keep] = w[keep]
    A, B, s = X.whitened_lowrank(E, wm, 3)
    assert np.all(A[np.setdiff1d(np.arange(11), keep)] == 0)
    A2, B2, s2 = X.whitened_lowrank(E[:, keep], w[keep], 3)
    assert np.allclose(s, s2, rtol=1e-12)
    assert np.allclose((A @ B)[keep], A2 @ B2, atol=1e-12)


def test_randomized_lowrank_exact_on_low_rank():
    rng = np.random.default_rng(5)
    U, sig, V, M = _known_svd(rng, 40, 30, [5, 4, 3, 2])
    w = rng.uniform(0.5, 2.0, 40)
    E = (M / w[:, None]).T
    omega = rng.standard_normal((30, 6))
    A, B, s = X.randomized_lowrank(E, w, omega, 4, 0)
    assert np.allclose(s, sig, rtol=1e-10)
    assert np.allclose(w[:, None] * (A @ B), M, atol=1e-10)


def test_randomized_lowrank_with_a_spectral_gap():
    # three large singular values over a small tail: one power iteration gives the truncated
    # SVD of the construction to high accuracy
    rng = np.random.default_rng(6)
    sig = [10, 9, 8] + [0.01] * 17
    U, sig, V, M = _known_svd(rng, 50, 25, sig)
    w = np.ones(50)
    omega = rng.standard_normal((25, 6))
    A, B, s = X.randomized_lowrank(M.T, w, omega, 3, 1)
    assert np.allclose(s, sig[:3], rtol=1e-7)
    assert np.allclose(A @ B, U[:, :3] @ np.diag(sig[:3]) @ V[:, :3].T, atol=1e-6)


def test_randomized_lowrank_never_beats_the_optimum():
    # flat spectrum: the randomized fit is never better than Eckart-Young's bound, and power
    # iterations bring it close
    rng = np.random.default_rng(7)
    E = rng.standard_normal((30, 40))
    w = rng.uniform(0.5, 2.0, 40)
    M = w[:, None] * E.T
    sv = np.linalg.svd(M, compute_uv=False)
    opt = np.sqrt(np.sum(sv[6:] ** 2))
    errs = []
    for q in (0, 3):
        A, B, _ = X.randomized_lowrank(E, w, rng.standard_normal((30, 10)), 6, q)
        errs.append(np.linalg.norm(M - w[:, None] * (A @ B)))
    assert errs[0] >= opt * (1 - 1e-12) and errs[1] >= opt * (1 - 1e-12)
    assert errs[1] <= opt * 1.05


def test_build_experts_structure():
    rng = np.random.default_rng(8)
    d_out, d_in, n_r, r_s, r_r, k = 24, 64, 3, 4, 3, 8
    W = (rng.standard_normal((d_out, d_in)) * 0.05).astype(np.float32)
    s = rng.uniform(0.5, 2.0, d_in).astype(np.float32)
    c = rng.uniform(0.2, 3.0, d_in)
    dep = np.array([3, 5, 8, 9, 13, 21, 22, 40, 41, 50, 60])
    labels = np.array([0, 0, 1, 2, 1, 0, 2, 1, 1, 2, 0])
    om = rng.standard_normal((1 + n_r, d_out, k))
    out = X.build_experts(W, s, 4, c, dep, labels, n_r, r_s, r_r, om, power_iters=6)
    E = X.quant_error(W, s, 4)
    # the SE removes (nearly) the top r_s whitened directions of E
    M = c[:, None] * E.T
    sv = np.linalg.svd(M, compute_uv=False)
    res_se = np.linalg.norm(c[:, None] * out["E1"].T)
    assert np.allclose(out["E1"], E - (out["A_s"] @ out["B_s"]).T)
    assert res_se <= np.sqrt(np.sum(sv[r_s:] ** 2)) * 1.02
    for g in range(n_r):
        ch = dep[labels == g]
        off = np.setdiff1d(np.arange(d_in), ch)
        assert np.all(out["A_r"][g][off] == 0)
        wg = np.zeros(d_in)
        wg[ch] = c[ch]
        before = np.linalg.norm(wg[:, None] * out["E1"].T)
        after = np.linalg.norm(wg[:, None] * (out["E1"].T - out["A_r"][g] @ out["B_r"][g]))
        assert after < before
        if len(ch) <= r_r:  # a cluster no wider than the rank is reconstructed exactly
            assert after < 1e-10 * before


def test_router_targets_hand_example():
    # one token x = [1, 2], E_1 = [[1, 0], [0, 1]] (so x E_1^T = [1, 2]); expert 0 reproduces E_1^T
    # exactly (A B = I): residual 0; expert 1 is zero: residual [1, 2], mean 1.5; expert 2 has
    # A B = [[0, 0], [0, 2]]: residual [1, 2 - 4] = [1, -2], mean 1.5 as well
    Xm = np.array([[1.0, 2.0]])
    E1 = np.eye(2)
    A = np.array([np.eye(2), np.zeros((2, 2)), np.diag([0.0, 2.0])])
    B = np.array([np.eye(2), np.zeros((2, 2)), np.eye(2)])
    assert np.allclose(X.router_targets(E1, Xm, A, B), [[0.0, 1.5, 1.5]])


def test_router_fit_recovers_a_consistent_system():
    # target = X R* exactly: with a vanishing ridge the fit returns R*; its gradient vanishes
    rng = np.random.default_rng(30)
    Xm = rng.standard_normal((200, 12))
    Rs = rng.standard_normal((12, 4))
    R = X.router_fit(Xm, Xm @ Rs, 1e-12)
    assert np.allclose(R, Rs, atol=1e-8)
    t = rng.standard_normal((200, 4))
    for ridge in (0.0, 0.1):
        R = X.router_fit(Xm, t, ridge)
        lam = ridge * np.sum(Xm * Xm) / 12
        grad = Xm.T @ (Xm @ R - t) + lam * R  # optimality of the ridge objective
        assert np.max(np.abs(grad)) < 1e-9 * np.max(np.abs(Xm.T @ t))
    # a large ridge shrinks the fit toward zero
    assert np.max(np.abs(X.router_fit(Xm, t, 1e6))) < 1e-5


def test_router_targets_rank_experts_by_their_residual():
    # an expert that removes part of E_1 leaves less error on every token than one that does not
    rng = np.random.default_rng(31)
    d_out, d_in = 10, 16
    E1 = rng.standard_normal((d_out, d_in))
    U, S, Vt = np.linalg.svd(E1.T, full_matrices=False)
    A = np.array([U[:, :4] * S[:4], np.zeros((d_in, 4))])
    B = np.array([Vt[:4], np.zeros((4, d_out))])
    Xm = rng.standard_normal((50, d_in))
    tg = X.router_targets(E1, Xm, A, B)
    assert np.all(tg[:, 0] < tg[:, 1])
    assert np.allclose(tg[:, 1], np.mean(np.abs(Xm @ E1.T), axis=1))


# ------------------------------------------------------------- covariance whitening
def _correlated(rng, T, n, rank_x=None):
    """Calibration tokens with strongly correlated channels: a few shared latent factors
    mixed into every channel, plus small independent noise and per-channel scales."""
    k = rank_x or max(2, n // 4)
    F = rng.standard_normal((T, k))
    M = rng.standard_normal((k, n))
    return (F @ M + 0.05 * rng.standard_normal((T, n))) * rng.uniform(0.2, 3.0, n)[None, :]


@pytest.mark.parametrize("d_out,n", [(40, 24), (24, 40)])  # both branches (n < d_out: thin QR)
def test_error_cov_lowrank_matches_svd_of_error_outputs(d_out, n):
    # Definition through the SVD of Z = E X^T: A_hat = U_r U_r^T E with U_r its left vectors
    rng = np.random.default_rng(21)
    E = rng.standard_normal((d_out, n))
    X = _correlated(rng, 60, n)
    r = 6
    A, B, sig = X_.error_cov_lowrank(E, X, r)
    U, S, _ = np.linalg.svd(E @ X.T)
    ref = U[:, :r] @ U[:, :r].T @ E
    assert np.allclose((A @ B).T, ref, atol=1e-9 * np.abs(ref).max())
    assert np.allclose(sig, S[:r], rtol=1e-9)


def test_error_cov_lowrank_equals_cholesky_whitened_svd():
    # The same minimizer derived the other way: whiten by L with L L^T = X^T X (the activation
    # second moment), truncate the SVD of E L, un-whiten: A_hat = [E L]_r L^-1.
    rng = np.random.default_rng(22)
    E = rng.standard_normal((30, 20))
    X = _correlated(rng, 200, 20, rank_x=20)
    r = 5
    A, B, _ = X_.error_cov_lowrank(E, X, r)
    L = np.linalg.cholesky(X.T @ X)
    U, S, Vt = np.linalg.svd(E @ L)
    ref = (U[:, :r] * S[:r]) @ Vt[:r] @ np.linalg.inv(L)
    assert np.allclose((A @ B).T, ref, atol=1e-8 * np.abs(ref).max())


def test_error_cov_lowrank_is_optimal_and_beats_diagonal_whitening():
    rng = np.random.default_rng(23)
    E = rng.standard_normal((48, 32))
    X = _correlated(rng, 300, 32, rank_x=6)
    r = 4
    A, B, sig = X_.error_cov_lowrank(E, X, r)
    res = X_.output_residual(E, X, A, B)
    # Eckart-Young: the residual is the energy of the dropped singular values of Z
    S = np.linalg.svd(E @ X.T, compute_uv=False)
    assert abs(res - np.sqrt(np.sum(S[r:] ** 2))) <= 1e-9 * res
    # no random rank-r perturbation of the factors does better
    for _ in range(50):
        Ap = A + 1e-3 * np.abs(A).max() * rng.standard_normal(A.shape)
        Bp = B + 1e-3 * np.abs(B).max() * rng.standard_normal(B.shape)
        assert X_.output_residual(E, X, Ap, Bp) >= res * (1 - 1e-12)
    # the diagonal (per-channel RMS) whitening ignores the correlations and must lose here
    Ad, Bd, _ = X_.whitened_lowrank(E, X_.channel_rms(X), r)
    assert X_.output_residual(E, X, Ad, Bd) > 1.05 * res


def test_error_cov_lowrank_full_rank_and_degenerate_cases():
    rng = np.random.default_rng(24)
    E = rng.standard_normal((20, 6))
    X = rng.standard_normal((50, 6))
    A, B, sig = X_.error_cov_lowrank(E, X, 8)  # rank above the number of channels
    assert np.allclose((A @ B).T, E, atol=1e-10)  # full recovery: the cluster case
    assert np.all(sig[6:] == 0) and np.all(sig[:6] > 0)
    A0, B0, s0 = X_.error_cov_lowrank(E, np.zeros((50, 6)), 3)  # no calibration energy
    assert not A0.any() and not B0.any() and not s0.any()


def test_build_experts_cov_structure():
    rng = np.random.default_rng(25)
    d_out, d_in, T = 24, 64, 200
    W = (rng.standard_normal((d_out, d_in)) * 0.05).astype(np.float32)
    s = rng.uniform(0.5, 2, d_in).astype(np.float32)
    X = _correlated(rng, T, d_in, rank_x=10)
    dep = np.array([3, 9, 10, 20, 33, 40, 41, 50, 51, 60])
    lab = np.array([0, 0, 1, 1, 1, 2, 2, 2, 0, 1])
    out = X_.build_experts_cov(W, s, 4, X, dep, lab, 3, 4, 8)
    E = X_.quant_error(W, s, 4)
    assert np.allclose(out["E1"], E - (out["A_s"] @ out["B_s"]).T)
    for g in range(3):
        ch = np.sort(dep[lab == g])
        others = np.setdiff1d(np.arange(d_in), ch)
        assert not out["A_r"][g][others].any()
        # clusters no wider than the rank are reproduced exactly on their channels
        rec = (out["A_r"][g][ch] @ out["B_r"][g]).T
        assert np.allclose(rec, out["E1"][:, ch], atol=1e-9)
    # the SE is the covariance-whitened fit of E itself
    A, B, _ = X_.error_cov_lowrank(E, X, 4)
    assert np.allclose(A @ B, out["A_s"] @ out["B_s"])
