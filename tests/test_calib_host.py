"""Host-side calibration steps of libqe (no GPU): the frequency partition and the NPMI /
spectral-embedding / K-Means clustering, compared with the oracle; argument checks of
the co-occurrence entry point that fail before any launch."""

import os

import numpy as np
import pytest

from oracle import qe_calib_oracle as C
from tests.test_oracle_calib import planted_topk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    lib_path = os.path.join(ROOT, "quantized_linear_moe_amd", "libqe.so")
    if not os.path.exists(lib_path):
        import importlib.util
        spec = importlib.util.spec_from_file_location("qe_build", os.path.join(ROOT, "quantized_linear_moe_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    from quantized_linear_moe_amd import _libqe
    return _libqe


@pytest.mark.parametrize("d_in,k,n_r,seed", [(8, 2, 2, 0), (4096, 32, 8, 1), (14336, 32, 8, 2), (300, 7, 5, 3)])
def test_partition_matches_oracle(L, d_in, k, n_r, seed):
    rng = np.random.default_rng(seed)
    hist = rng.integers(0, 40, d_in).astype(np.uint32)  # many ties
    indep, dep, slot = L.qe_partition_channels(hist, k, n_r)
    oi, od = C.frequency_partition(hist, k, n_r)
    np.testing.assert_array_equal(indep, oi)
    np.testing.assert_array_equal(dep, od)
    expect = np.full(d_in, -1, np.int32)
    expect[od] = np.arange(len(od))
    np.testing.assert_array_equal(slot, expect)


def test_partition_argument_errors(L):
    lib = L.raw_library()
    hist = np.zeros(16, np.uint32)
    buf = np.zeros(64, np.int32)
    assert lib.qe_partition_channels(hist.ctypes.data, 16, 4, 4, buf.ctypes.data, buf.ctypes.data, None) == \
        L.QE_ERR_INVALID_ARG  # 4 * (1 + 4) > 16
    assert lib.qe_partition_channels(hist.ctypes.data, 16, 0, 2, buf.ctypes.data, buf.ctypes.data, None) == \
        L.QE_ERR_INVALID_ARG
    assert lib.qe_partition_channels(None, 16, 2, 2, buf.ctypes.data, buf.ctypes.data, None) == L.QE_ERR_INVALID_ARG


def test_cooccur_argument_errors_before_launch(L):
    lib = L.raw_library()
    need = L.qe_cooccur_workspace_bytes(1000, 256)
    assert need == 32 * 256 * 4  # 1000 tokens: 32 mask words of 32 tokens (whole 128-token chunks) per channel
    assert L.qe_cooccur_workspace_bytes(1000, 8193) == 0 and L.qe_cooccur_workspace_bytes(-1, 16) == 0
    ws = 1 << 20
    assert lib.qe_cooccur(None, 0, 8, None, 64, 16, None, None, 0, None) == L.QE_OK  # T == 0: no-op
    assert lib.qe_cooccur(4096, 4, 65, 8192, 64, 16, 8192, ws, need, None) == L.QE_ERR_INVALID_ARG  # k > d_in
    assert lib.qe_cooccur(4096, 4, 0, 8192, 64, 16, 8192, ws, need, None) == L.QE_ERR_INVALID_ARG
    assert lib.qe_cooccur(4096, 4, 8, 8192, 64, 0, 8192, ws, need, None) == L.QE_ERR_INVALID_ARG
    assert lib.qe_cooccur(4096, 4, 8, 8192, 64, 8193, 8192, ws, need, None) == L.QE_ERR_UNSUPPORTED
    assert lib.qe_cooccur(4096, 4, 1025, 8192, 4096, 16, 8192, ws, need, None) == L.QE_ERR_UNSUPPORTED
    assert lib.qe_cooccur(4100, 4, 8, 8192, 64, 16, 8192, ws, need, None) == L.QE_ERR_ALIGNMENT
    assert lib.qe_cooccur(4096, 4, 8, None, 64, 16, 8192, ws, need, None) == L.QE_ERR_INVALID_ARG
    small = L.qe_cooccur_workspace_bytes(1000, 16)
    assert lib.qe_cooccur(4096, 1000, 8, 8192, 64, 16, 8192, ws, small - 1, None) == L.QE_ERR_WORKSPACE
    assert lib.qe_cooccur(4096, 1000, 8, 8192, 64, 16, 8192, None, small, None) == L.QE_ERR_WORKSPACE
    assert lib.qe_cooccur(4096, 1000, 8, 8192, 64, 16, 8192, ws + 8, small, None) == L.QE_ERR_ALIGNMENT


def test_cluster_argument_errors(L):
    lib = L.raw_library()
    good = np.array([[3, 1], [1, 2]], np.uint32)
    lab = np.zeros(2, np.int32)

    def call(c, n=2, T=4, K=2, thr=0.2):
        c = np.ascontiguousarray(c, np.uint32)
        return lib.qe_cluster_channels(c.ctypes.data, n, T, K, thr, lab.ctypes.data, None, None, None)

    assert call(good) == L.QE_OK
    assert call(np.array([[3, 1], [0, 2]])) == L.QE_ERR_INVALID_ARG  # not symmetric
    assert call(np.array([[3, 3], [3, 2]])) == L.QE_ERR_INVALID_ARG  # pair count above a channel count
    assert call(good, T=2) == L.QE_ERR_INVALID_ARG  # channel count above T
    assert call(good, K=3) == L.QE_ERR_INVALID_ARG
    assert call(good, K=0) == L.QE_ERR_INVALID_ARG
    assert call(good, thr=-0.1) == L.QE_ERR_INVALID_ARG
    assert call(good, thr=float("nan")) == L.QE_ERR_INVALID_ARG
    assert call(good, T=0) == L.QE_ERR_INVALID_ARG
    assert lib.qe_cluster_channels(good.ctypes.data, 2049, 4, 2, 0.2, lab.ctypes.data, None, None, None) == \
        L.QE_ERR_UNSUPPORTED


def _compare_clustering(L, cooc, T, K, thr, labels_equal=True):
    got, S, ev, U = L.qe_cluster_channels(cooc, T, K, thr, outputs=True)
    o_lab, o_S, o_U, o_ev = C.cluster_channels(cooc, T, K, thr)
    np.testing.assert_allclose(S, o_S, rtol=0, atol=1e-13)
    np.testing.assert_allclose(ev, o_ev, rtol=0, atol=1e-10)
    # the embedding is unique up to an orthogonal map of the eigenspace: compare its Gram matrix
    np.testing.assert_allclose(U @ U.T, o_U @ o_U.T, rtol=0, atol=1e-8)
    assert got.min() >= 0 and got.max() < K
    if labels_equal:
        np.testing.assert_array_equal(got, o_lab)
    return got, o_lab


@pytest.mark.parametrize("cross_prob", [0.0, 0.05])
def test_cluster_matches_oracle_on_planted_groups(L, cross_prob):
    rng = np.random.default_rng(11)
    d_in, k, n_r, T = 96, 8, 3, 900
    topk, always, groups = planted_topk(T, d_in, k, n_r, rng, cross_prob)
    hist = np.bincount(topk.reshape(-1), minlength=d_in)
    _, dep = C.frequency_partition(hist, k, n_r)
    cooc = C.cooccurrence(topk, dep, d_in).astype(np.uint32)
    got, o_lab = _compare_clustering(L, cooc, T, n_r, 0.2)
    group_of = {int(c): g for g, gs in enumerate(groups) for c in gs}
    np.testing.assert_array_equal(got, C.canonical_labels(np.array([group_of[int(c)] for c in dep])))


def test_cluster_matches_oracle_at_the_pages_settings(L):
    # N_r = 8 routed experts of k = 32 channels each: 256 token-dependent channels
    rng = np.random.default_rng(7)
    d_in, k, n_r, T = 4096, 32, 8, 4096
    topk, _, groups = planted_topk(T, d_in, k, n_r, rng, cross_prob=0.1)
    hist = np.bincount(topk.reshape(-1), minlength=d_in)
    _, dep = C.frequency_partition(hist, k, n_r)
    cooc = C.cooccurrence(topk, dep, d_in).astype(np.uint32)
    got, o_lab = _compare_clustering(L, cooc, T, n_r, 0.2)
    group_of = {int(c): g for g, gs in enumerate(groups) for c in gs}
    np.testing.assert_array_equal(got, C.canonical_labels(np.array([group_of[int(c)] for c in dep])))


def test_cluster_on_unstructured_counts(L):
    # top-k sets of random activations have no planted structure: the similarity and the
    # spectrum still agree with the oracle; the labels agree too unless K-Means meets a
    # near-tie, in which case both must be Lloyd fixed points of their own embedding
    rng = np.random.default_rng(4)
    from oracle import qe_oracle as O
    x = rng.standard_normal((2048, 512)).astype(np.float32)
    w = np.abs(rng.standard_normal(512)).astype(np.float32)
    topk, hist = O.channel_topk(x, w, 16)
    _, dep = C.frequency_partition(hist, 16, 4)
    cooc = C.cooccurrence(topk, dep, 512).astype(np.uint32)
    for thr in (0.0, 0.05):
        got, S, ev, U = L.qe_cluster_channels(cooc, 2048, 4, thr, outputs=True)
        o_lab, o_S, o_U, o_ev = C.cluster_channels(cooc, 2048, 4, thr)
        np.testing.assert_allclose(S, o_S, rtol=0, atol=1e-13)
        np.testing.assert_allclose(ev, o_ev, rtol=0, atol=1e-10)
        if not np.array_equal(got, o_lab):
            for lab, emb in ((got, U), (o_lab, o_U)):
                cent = np.stack([emb[lab == c].mean(axis=0) for c in range(lab.max() + 1)])
                d = ((emb[:, None, :] - cent[None]) ** 2).sum(axis=2)
                assert (d[np.arange(len(lab)), lab] <= d.min(axis=1) + 1e-12).all()


@pytest.mark.parametrize("n", [1, 2, 3, 17, 64])
def test_eigen_solver_small_and_degenerate(L, n):
    # through the cluster entry point: co-occurrence of channels that always appear together
    # (one component, all NPMI = 1) and of disjoint channels (identity similarity: eigenvalue
    # 0 with multiplicity n)
    T = 50
    together = np.full((n, n), 10, np.uint32)
    lab, S, ev, U = L.qe_cluster_channels(together, T, 1, 0.2, outputs=True)
    assert lab.tolist() == [0] * n and abs(ev[0]) < 1e-12
    disjoint = np.diag(np.full(n, 5, np.uint32))
    K = min(n, 3)
    lab, S, ev, U = L.qe_cluster_channels(disjoint, T, K, 0.2, outputs=True)
    np.testing.assert_allclose(ev, 0.0, atol=1e-12)
    np.testing.assert_allclose(S, np.eye(n), atol=0)
