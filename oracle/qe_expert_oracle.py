"""CPU oracle for the construction of the QE experts (post-training, before inference).

Test infrastructure only: tests, the smoke check and the benchmark's CPU baseline import it;
the library never does.  fp64 throughout, numpy's QR / SVD as library primitives.

Sources (pages as titles, with the section each step follows):
  * MCISLAB DeepRead summary of "Quant Experts", section "Method", Shared Expert (SE): the
    layer's quantization error is E = W_f - W_q; the SE is a low-rank reconstruction of it,
    with channel-wise scaling of the activations.  Routed Experts (REs): the error left after
    the SE goes to the REs, one low-rank adapter per cluster of token-dependent channels.
    Section "Experiments": total rank r = 64 split evenly between SE and REs, k = 32, N_r = 8.
  * PaperDaily post "西交大提出Quant Experts：token级量化补偿", section "核心设计": the SE
    reconstructs the error by a whitening SVD, which balances the scales of the directions
    before the decomposition so the low-rank factors capture the dominant error.
  * Halko, Martinsson and Tropp, "Finding structure with randomness" (SIAM Review 2011),
    Algorithm 4.4 (randomized subspace iteration) and Algorithm 5.1 (direct SVD of the
    small matrix): the randomized truncated SVD, with the Gaussian test matrix an input.

Readings where the pages leave a step open (each also listed in the design notes):
  * W_q is the effective quantized weight in the input domain of x: the codes of
    W_f * diag(s) times the row scale, divided by s (the adapters act on x, not x / s).
  * Whitening is diagonal: input channel j is weighted by the RMS of its calibration
    activations, c_j = sqrt(mean_t x[t, j]^2), so the SVD of M = diag(c) E^T minimizes the
    expected output error sum_t |x_t (E^T - A B)|^2 under a diagonal activation covariance;
    A = diag(1/c) U_r S_r^(1/2) (rows with c_j = 0 are zero), B = S_r^(1/2) V_r^T.
  * The SE approximates the whole E; the RE of cluster g approximates the residual
    E_1 = E - (A_s B_s)^T on the input channels of that cluster only (weights c_j on the
    cluster, 0 elsewhere), so its A rows outside the cluster are zero.
  * The router predicts, for each routed expert, the error that would remain on a token if that
    expert were used, and the token takes the expert with the smallest prediction (DeepRead,
    "Method", REs; WisPaper post "[CVPR 2025] Quant Experts: Adapting PTQ to the Heterogeneity
    of Vision-Language Tokens", section "Critical Analysis & Insight": a prediction of the absolute mean
    error).  Its target for token t and expert g is the mean absolute residual over the
    output channels, mean_i |x_t (E_1^T - A_g B_g)|_i, and R is the ridge least-squares fit
    (X^T X + lam I) R = X^T target with lam = ridge * trace(X^T X) / d_in.
Covariance-whitened construction (the reading the library's default expert build follows):
  * PaperDaily "核心设计" states the objective: the original error, minus the shared expert's
    and the routed expert's compensation, multiplied by the input token, should leave the
    smallest residual; and the whitening computes a covariance and whitens with it so that
    the SVD captures the error's main components instead of directions that are merely
    large.  The plain reading: the SE is the rank-r_s minimizer of
    sum_t |(E - A_hat) x_t|^2 over the calibration tokens, and the covariance is that of the
    error outputs E x_t: C = sum_t (E x_t)(E x_t)^T = Z Z^T with Z = E X^T.  By Eckart-Young
    on Z, A_hat = U_r U_r^T E with U_r the top-r eigenvectors of C (A_hat X^T = U_r U_r^T Z is
    then the best rank-r approximation of Z).  This is the same subspace as the SVD of E L
    with L L^T = X^T X (whitening by the activation second moment); the pins check both.
    Factors: A = E^T U_r [d_in, r], B = U_r^T [r, d_out], so x A B = x A_hat^T.
  * The RE of cluster g minimizes the same objective for the residual E_1 = E - A_hat_s on
    the cluster's input channels only: E_1[:, C_g] with the tokens' values on C_g.
  * Eigen-directions below 1e-12 of the largest eigenvalue are dropped (zero columns), so
    a cluster no wider than the rank reproduces E_1[:, C_g] exactly.
parity pinned: every function below has CPU pins in tests/test_oracle_experts.py.
"""

from typing import Dict, Optional, Sequence, Tuple

import numpy as np

from . import qe_oracle as O


def quant_error(W_f: np.ndarray, s: Optional[np.ndarray], w_bits: int) -> np.ndarray:
    """E = W_f - W_q with W_q = diag(s_w) q diag(1/s) ([DeepRead] "Method", SE).

    The codes and row scales are the weight quantizer's (float32 decisions); E in fp64.
    """
    q, s_w = O.quant_weights(W_f, s, w_bits)
    Wq = s_w.astype(np.float64)[:, None] * q.astype(np.float64)
    if s is not None:
        Wq = Wq / np.asarray(s, dtype=np.float64)[None, :]
    return np.asarray(W_f, dtype=np.float64) - Wq


def channel_rms(x: np.ndarray) -> np.ndarray:
    """Whitening weights c_j = sqrt(mean_t x[t, j]^2) over the calibration tokens."""
    x = np.asarray(x, dtype=np.float64)
    return np.sqrt(np.mean(x * x, axis=0))


def _factors(U: np.ndarray, S: np.ndarray, Vt: np.ndarray, w: np.ndarray, r: int):
    """A = diag(1/w) U_r S_r^(1/2) (zero rows where w = 0), B = S_r^(1/2) V_r^T."""
    root = np.sqrt(S[:r])
    inv = np.zeros_like(w, dtype=np.float64)
    nz = w > 0
    inv[nz] = 1.0 / w[nz]
    A = inv[:, None] * U[:, :r] * root[None, :]
    B = root[:, None] * Vt[:r, :]
    return A, B, S[:r].copy()


def whitened_lowrank(E: np.ndarray, w: np.ndarray, r: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """The definition: truncated SVD of M = diag(w) E^T, rank r (Eckart-Young optimal).

    Returns A [d_in, r], B [r, d_out] with diag(w) A B = M_r, and the r singular values.
    """
    M = np.asarray(w, dtype=np.float64)[:, None] * np.asarray(E, dtype=np.float64).T
    U, S, Vt = np.linalg.svd(M, full_matrices=False)
    return _factors(U, S, Vt, np.asarray(w, dtype=np.float64), r)


def randomized_lowrank(E: np.ndarray, w: np.ndarray, omega: np.ndarray, r: int,
                       power_iters: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Randomized truncated SVD of M = diag(w) E^T with test matrix omega [d_out, k], k >= r.

    Halko-Martinsson-Tropp Algorithm 4.4: Y = M omega, Q = qr(Y); power_iters times
    (Q~ = qr(M^T Q), Q = qr(M Q~)); then Algorithm 5.1: B = Q^T M, B = U~ S V^T, U = Q U~.
    """
    M = np.asarray(w, dtype=np.float64)[:, None] * np.asarray(E, dtype=np.float64).T
    Q, _ = np.linalg.qr(M @ np.asarray(omega, dtype=np.float64))
    for _ in range(power_iters):
        Qt, _ = np.linalg.qr(M.T @ Q)
        Q, _ = np.linalg.qr(M @ Qt)
    Bsmall = Q.T @ M
    Ut, S, Vt = np.linalg.svd(Bsmall, full_matrices=False)
    return _factors(Q @ Ut, S, Vt, np.asarray(w, dtype=np.float64), r)


def build_experts(W_f: np.ndarray, s: Optional[np.ndarray], w_bits: int, c: np.ndarray,
                  dep_channels: Sequence[int], labels: Sequence[int], n_r: int, r_s: int, r_r: int,
                  omegas: np.ndarray, power_iters: int) -> Dict[str, np.ndarray]:
    """SE and REs of one linear ([DeepRead] "Method": SE first, the residual to the REs).

    c: whitening weights [d_in]; dep_channels / labels: the token-dependent channels and
    their cluster in [0, n_r); omegas [1 + n_r, d_out, k]: the test matrix of the SE fit,
    then of each RE fit.  Returns A_s [d_in, r_s], B_s [r_s, d_out], A_r [n_r, d_in, r_r],
    B_r [n_r, r_r, d_out], sigma_s, sigma_r, and the residual error E_1 [d_out, d_in].
    """
    E = quant_error(W_f, s, w_bits)
    c = np.asarray(c, dtype=np.float64)
    d_out, d_in = E.shape
    out: Dict[str, np.ndarray] = {}
    if r_s > 0:
        A_s, B_s, sig_s = randomized_lowrank(E, c, omegas[0], r_s, power_iters)
        E1 = E - (A_s @ B_s).T
    else:
        A_s, B_s, sig_s = np.zeros((d_in, 0)), np.zeros((0, d_out)), np.zeros(0)
        E1 = E
    A_r = np.zeros((n_r, d_in, r_r))
    B_r = np.zeros((n_r, r_r, d_out))
    sig_r = np.zeros((n_r, r_r))
    dep = np.asarray(dep_channels, dtype=np.int64)
    lab = np.asarray(labels, dtype=np.int64)
    for g in range(n_r):
        wg = np.zeros(d_in)
        ch = dep[lab == g]
        wg[ch] = c[ch]
        A_r[g], B_r[g], sig_r[g] = randomized_lowrank(E1, wg, omegas[1 + g], r_r, power_iters)
    out.update(A_s=A_s, B_s=B_s, sigma_s=sig_s, A_r=A_r, B_r=B_r, sigma_r=sig_r, E1=E1)
    return out


def router_targets(E1: np.ndarray, X: np.ndarray, A_r: np.ndarray, B_r: np.ndarray) -> np.ndarray:
    """target[t, g] = mean_i |x_t (E_1^T - A_g B_g)|_i: the error expert g leaves on token t."""
    X = np.asarray(X, dtype=np.float64)
    base = X @ np.asarray(E1, dtype=np.float64).T
    out = np.empty((X.shape[0], A_r.shape[0]))
    for g in range(A_r.shape[0]):
        res = base - (X @ np.asarray(A_r[g], dtype=np.float64)) @ np.asarray(B_r[g], dtype=np.float64)
        out[:, g] = np.mean(np.abs(res), axis=1)
    return out


def router_fit(X: np.ndarray, target: np.ndarray, ridge: float) -> np.ndarray:
    """Ridge least squares: R = (X^T X + lam I)^-1 X^T target, lam = ridge * trace(X^T X) / d_in."""
    X = np.asarray(X, dtype=np.float64)
    G = X.T @ X
    lam = ridge * np.trace(G) / X.shape[1]
    return np.linalg.solve(G + lam * np.eye(X.shape[1]), X.T @ np.asarray(target, dtype=np.float64))


# ------------------------------------------------------------------ covariance whitening
def error_cov_lowrank(E: np.ndarray, X: np.ndarray, r: int, tol: float = 1e-12
                      ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Rank-r minimizer of sum_t |(E - A_hat) x_t|^2 (PaperDaily "核心设计").

    E [d_out, n] (the error on n input channels), X [T, n] (calibration tokens on those
    channels).  U_r = top-r eigenvectors of the error-output covariance C = Z Z^T, Z = E X^T;
    A_hat = U_r U_r^T E.  Returns A = E^T U_r [n, r], B = U_r^T [r, d_out] and the singular
    values of Z (sqrt of the top-r eigenvalues, 0 for dropped directions), descending.
    When n < d_out the eigenproblem is reduced exactly through a thin QR of E (range(Z) lies
    in range(E)): E = Q R, C = Q (R X^T X R^T) Q^T.
    """
    E = np.asarray(E, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    d_out, n = E.shape
    if n < d_out:
        Qe, Re = np.linalg.qr(E)
        Zs = Re @ X.T
        lam, W = np.linalg.eigh(Zs @ Zs.T)
        U = Qe @ W
    else:
        Z = E @ X.T
        lam, U = np.linalg.eigh(Z @ Z.T)
    order = np.argsort(lam)[::-1][:r]
    lam, U = lam[order], U[:, order]
    top = max(float(lam[0]) if len(lam) else 0.0, 0.0)
    keep = lam > tol * top if top > 0 else np.zeros(len(lam), bool)
    U = np.where(keep[None, :], U, 0.0)
    sig = np.where(keep, np.sqrt(np.maximum(lam, 0.0)), 0.0)
    if U.shape[1] < r:  # fewer directions than the rank
        U = np.concatenate([U, np.zeros((d_out, r - U.shape[1]))], axis=1)
        sig = np.concatenate([sig, np.zeros(r - len(sig))])
    return E.T @ U, U.T.copy(), sig


def output_residual(E: np.ndarray, X: np.ndarray, A: np.ndarray, B: np.ndarray) -> float:
    """sqrt(sum_t |(E - (A B)^T) x_t|^2) = |X E^T - X A B|_F."""
    X = np.asarray(X, dtype=np.float64)
    return float(np.linalg.norm(X @ np.asarray(E, np.float64).T - (X @ np.asarray(A, np.float64)) @ B))


def build_experts_cov(W_f: np.ndarray, s: Optional[np.ndarray], w_bits: int, X: np.ndarray,
                      dep_channels: Sequence[int], labels: Sequence[int], n_r: int, r_s: int, r_r: int
                      ) -> Dict[str, np.ndarray]:
    """SE and REs by covariance whitening ([DeepRead] "Method": the SE first, the residual to
    the REs, one per cluster; [PaperDaily] "核心设计": the residual-times-token objective).

    X [T, d_in]: calibration tokens (the layer input the adapters read, bf16 values).
    Returns A_s, B_s, sigma_s, A_r [n_r, d_in, r_r] (zero outside the cluster's channels),
    B_r, sigma_r and E1 = E - (A_s B_s)^T.
    """
    E = quant_error(W_f, s, w_bits)
    X = np.asarray(X, dtype=np.float64)
    d_out, d_in = E.shape
    if r_s > 0:
        A_s, B_s, sig_s = error_cov_lowrank(E, X, r_s)
        E1 = E - (A_s @ B_s).T
    else:
        A_s, B_s, sig_s = np.zeros((d_in, 0)), np.zeros((0, d_out)), np.zeros(0)
        E1 = E
    A_r = np.zeros((n_r, d_in, r_r))
    B_r = np.zeros((n_r, r_r, d_out))
    sig_r = np.zeros((n_r, r_r))
    dep = np.asarray(dep_channels, dtype=np.int64)
    lab = np.asarray(labels, dtype=np.int64)
    for g in range(n_r):
        ch = np.sort(dep[lab == g])
        if len(ch) == 0:
            continue
        Ag, B_r[g], sig_r[g] = error_cov_lowrank(E1[:, ch], X[:, ch], r_r)
        A_r[g][ch] = Ag
    return dict(A_s=A_s, B_s=B_s, sigma_s=sig_s, A_r=A_r, B_r=B_r, sigma_r=sig_r, E1=E1)
