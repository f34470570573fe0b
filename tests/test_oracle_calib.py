"""Pins of the calibration-statistic oracle (frequency partition, co-occurrence, NPMI,
normalized-Laplacian spectral embedding, K-Means) against facts that do not come from
the oracle itself: hand-worked cases, brute-force counting, spectral properties of
graphs with known structure, and planted channel groups that must be recovered."""

import numpy as np
import pytest

from oracle import qe_calib_oracle as C
from oracle import qe_oracle as O


# ----------------------------------------------------------------- frequency partition
def test_frequency_partition_hand_worked():
    # counts:        ch0 ch1 ch2 ch3 ch4 ch5 ch6 ch7
    hist = np.array([5, 9, 9, 0, 3, 9, 1, 3])
    # by count desc, index asc: 1, 2, 5 (9); 0 (5); 4, 7 (3); 6 (1); 3 (0)
    indep, dep = C.frequency_partition(hist, k=2, n_r=2)
    assert indep.tolist() == [1, 2]
    assert dep.tolist() == [5, 0, 4, 7]
    indep, dep = C.frequency_partition(hist, k=1, n_r=7)
    assert indep.tolist() == [1] and dep.tolist() == [2, 5, 0, 4, 7, 6, 3]
    with pytest.raises(ValueError):
        C.frequency_partition(hist, k=2, n_r=4)


# ----------------------------------------------------------------- co-occurrence counts
def _brute_cooccurrence(topk, dep):
    n = len(dep)
    out = np.zeros((n, n), np.int64)
    sets = [set(int(c) for c in row) for row in topk]
    for i in range(n):
        for j in range(n):
            out[i, j] = sum(1 for s in sets if int(dep[i]) in s and int(dep[j]) in s)
    return out


@pytest.mark.parametrize("T,k,d,n_r", [(1, 3, 20, 2), (37, 5, 40, 3), (64, 8, 48, 4)])
def test_cooccurrence_brute_force(T, k, d, n_r):
    rng = np.random.default_rng(T * 7 + k)
    topk = np.stack([rng.choice(d, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    hist = np.bincount(topk.reshape(-1), minlength=d)
    _, dep = C.frequency_partition(hist, k, n_r)
    got = C.cooccurrence(topk, dep, d)
    np.testing.assert_array_equal(got, _brute_cooccurrence(topk, dep))
    assert np.array_equal(got, got.T)
    np.testing.assert_array_equal(np.diag(got), hist[dep])


def test_cooccurrence_diagonal_is_the_topk_histogram():
    # the diagonal counts how often each token-dependent channel was selected: the a8 histogram
    rng = np.random.default_rng(5)
    x = rng.standard_normal((96, 64)).astype(np.float32)
    w = np.abs(rng.standard_normal(64)).astype(np.float32)
    topk, hist = O.channel_topk(x, w, 6)
    indep, dep = C.frequency_partition(hist, 6, 3)
    cooc = C.cooccurrence(topk, dep, 64)
    np.testing.assert_array_equal(np.diag(cooc), hist[dep])
    assert (cooc <= np.minimum.outer(np.diag(cooc), np.diag(cooc))).all()


# ----------------------------------------------------------------- NPMI
def test_npmi_hand_worked():
    # 4 tokens: {a, b}, {a}, {b}, {}  ->  p(a) = p(b) = 1/2, p(a,b) = 1/4 = p(a) p(b): independent
    S = C.npmi(np.array([[2, 1], [1, 2]]), 4)
    assert S[0, 1] == 0.0 and S[1, 0] == 0.0
    assert S[0, 0] == pytest.approx(1.0, abs=1e-15) and S[1, 1] == pytest.approx(1.0, abs=1e-15)
    # always together (p = 1/2 each): ln(2)/ln(2) = 1; never together: -1
    assert C.npmi(np.array([[2, 2], [2, 2]]), 4)[0, 1] == pytest.approx(1.0, abs=1e-15)
    assert C.npmi(np.array([[2, 0], [0, 2]]), 4)[0, 1] == -1.0
    # in every token: the p = 1 limit
    assert C.npmi(np.array([[4, 4], [4, 4]]), 4)[0, 1] == 1.0
    # T = 10, p(a) = 0.5, p(b) = 0.4, p(a,b) = 0.3: ln(1.5) / ln(10/3) = 0.33677264689975...
    v = C.npmi(np.array([[5, 3], [3, 4]]), 10)
    assert v[0, 1] == pytest.approx(0.3367726468997534, rel=1e-14)
    # a channel that never occurs: -1 on its row, column and diagonal
    z = C.npmi(np.array([[5, 0], [0, 0]]), 10)
    assert z[1].tolist() == [-1.0, -1.0] and z[0, 1] == -1.0


def test_similarity_threshold():
    cooc = np.array([[5, 3, 0, 1], [3, 4, 2, 0], [0, 2, 6, 0], [1, 0, 0, 1]])
    raw = C.npmi(cooc, 10)
    S = C.similarity(cooc, 10, threshold=0.2)
    assert S[0, 1] == pytest.approx(0.3367726468997534, rel=1e-14)
    # p(0) = 0.5, p(3) = 0.1, p(0,3) = 0.1: ln 2 / ln 10 = log10(2), kept
    assert S[0, 3] == pytest.approx(0.30102999566398120, rel=1e-14)
    # p(1) = 0.4, p(2) = 0.6, p(1,2) = 0.2: ln(5/6) / ln 5 = -0.1133, dropped; never together: dropped
    assert raw[1, 2] == pytest.approx(-0.11328275255937, rel=1e-12) and S[1, 2] == 0.0
    assert raw[0, 2] == -1.0 and S[0, 2] == 0.0
    assert (S[raw < 0.2] == 0).all() and (S[raw >= 0.2] == raw[raw >= 0.2]).all()
    assert (np.abs(raw) <= 1.0 + 1e-12).all() and np.array_equal(raw, raw.T)
    with pytest.raises(ValueError):
        C.similarity(cooc, 10, threshold=-0.1)


# ----------------------------------------------------------------- spectral embedding
def _block_diagonal(sizes, rng):
    n = sum(sizes)
    S = np.zeros((n, n))
    o = 0
    for s in sizes:
        B = rng.uniform(0.3, 1.0, (s, s))
        S[o:o + s, o:o + s] = (B + B.T) / 2
        o += s
    return S


def test_spectral_disconnected_components():
    # the multiplicity of eigenvalue 0 of the normalized Laplacian is the number of
    # connected components; the normalized embedding maps each component to one point,
    # and points of different components are orthogonal
    rng = np.random.default_rng(1)
    sizes = [3, 4, 5]
    S = _block_diagonal(sizes, rng)
    perm = rng.permutation(S.shape[0])
    S = S[np.ix_(perm, perm)]
    comp = np.repeat(np.arange(3), sizes)[perm]
    U, w = C.spectral_embedding(S, 3)
    assert np.abs(w).max() < 1e-12
    _, w4 = C.spectral_embedding(S, 4)
    assert w4[3] > 1e-3
    G = U @ U.T
    same = comp[:, None] == comp[None, :]
    np.testing.assert_allclose(G[same], 1.0, atol=1e-10)
    np.testing.assert_allclose(G[~same], 0.0, atol=1e-10)


def test_spectral_textbook_spectrum():
    rng = np.random.default_rng(2)
    n = 12
    B = rng.uniform(0.0, 1.0, (n, n))
    S = (B + B.T) / 2  # connected: every weight positive
    _, w = C.spectral_embedding(S, n)
    assert abs(w[0]) < 1e-12 and w[1] > 1e-6
    assert w.min() > -1e-12 and w.max() < 2 + 1e-12
    # a bipartite graph (even cycle, no self loops) has eigenvalue exactly 2
    cyc = np.zeros((8, 8))
    for i in range(8):
        cyc[i, (i + 1) % 8] = cyc[(i + 1) % 8, i] = 1.0
    _, wc = C.spectral_embedding(cyc, 8)
    assert wc[-1] == pytest.approx(2.0, abs=1e-12)
    # cycle of 8: eigenvalues 1 - cos(2 pi m / 8)
    ref = np.sort(1 - np.cos(2 * np.pi * np.arange(8) / 8))
    np.testing.assert_allclose(wc, ref, atol=1e-12)


# ----------------------------------------------------------------- K-Means
def test_kmeans_hand_worked():
    # seeds: row 0 (x=0) and the farthest row (x=20); x=10 is equidistant and goes to the
    # lower cluster first, then moves to the right cluster once the centroids update
    U = np.array([[0.0], [1.0], [10.0], [11.0], [20.0]])
    assert C.kmeans(U, 2).tolist() == [0, 0, 1, 1, 1]
    assert C.kmeans(U, 1).tolist() == [0] * 5
    assert C.kmeans(U, 5).tolist() == [0, 1, 2, 3, 4]


def test_kmeans_recovers_blobs_and_is_a_fixed_point():
    rng = np.random.default_rng(3)
    centers = np.array([[0.0, 0.0], [10.0, 0.0], [0.0, 10.0], [10.0, 10.0]])
    planted = np.repeat(np.arange(4), 15)
    rng.shuffle(planted)
    U = centers[planted] + rng.normal(0, 0.5, (planted.size, 2))
    labels = C.kmeans(U, 4)
    np.testing.assert_array_equal(labels, C.canonical_labels(planted))
    # Lloyd fixed point: every point is nearest to its own cluster's mean
    cent = np.stack([U[labels == c].mean(axis=0) for c in range(4)])
    d = ((U[:, None, :] - cent[None]) ** 2).sum(axis=2)
    np.testing.assert_array_equal(np.argmin(d, axis=1), labels)


def test_canonical_labels():
    assert C.canonical_labels(np.array([3, 3, 1, 0, 1, 2])).tolist() == [0, 0, 1, 2, 1, 3]


# ----------------------------------------------------------------- planted channel groups
def planted_topk(T, d_in, k, n_groups, rng, cross_prob=0.0):
    """Tokens whose top-k sets hold half 'always-on' channels and half channels of one
    group; returns (topk [T, k], always-on channels, group channel lists)."""
    chans = rng.permutation(d_in)
    always = chans[:k]
    groups = [chans[k + g * k: k + (g + 1) * k] for g in range(n_groups)]
    rows = []
    half = k // 2
    for _ in range(T):
        g = rng.integers(n_groups)
        a = rng.choice(always, size=k - half, replace=False)
        b = rng.choice(groups[g], size=half, replace=False)
        if cross_prob and rng.random() < cross_prob:
            other = groups[(g + 1 + rng.integers(n_groups - 1)) % n_groups]
            extra = [c for c in rng.permutation(other) if c not in b][:1]
            a = np.concatenate([a[:-1], extra])
        rows.append(np.concatenate([a, b]))
    return np.stack(rows).astype(np.int32), always, groups


@pytest.mark.parametrize("cross_prob", [0.0, 0.05])
def test_cluster_channels_recovers_planted_groups(cross_prob):
    rng = np.random.default_rng(11)
    d_in, k, n_r, T = 96, 8, 3, 900
    topk, always, groups = planted_topk(T, d_in, k, n_r, rng, cross_prob)
    hist = np.bincount(topk.reshape(-1), minlength=d_in)
    indep, dep = C.frequency_partition(hist, k, n_r)
    assert set(indep.tolist()) == set(always.tolist())
    group_of = {int(c): g for g, gs in enumerate(groups) for c in gs}
    assert set(dep.tolist()) == set(group_of)
    cooc = C.cooccurrence(topk, dep, d_in)
    labels, S, U, w = C.cluster_channels(cooc, T, n_r, 0.2)
    truth = C.canonical_labels(np.array([group_of[int(c)] for c in dep]))
    np.testing.assert_array_equal(labels, truth)
    assert S.shape == (n_r * k, n_r * k) and U.shape == (n_r * k, n_r) and w.shape == (n_r,)
