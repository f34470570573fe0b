"""GPU parity of the co-occurrence counts (bit-exact against the oracle) and of the whole
calibration chain: per-token top-k -> frequency partition -> co-occurrence -> NPMI
spectral clustering, on seeded synthetic activations with planted channel groups."""

import numpy as np
import pytest
import torch

from oracle import qe_calib_oracle as C
from oracle import qe_oracle as O
from tests.test_oracle_calib import planted_topk

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def Q():
    import quantized_linear_moe_amd as q
    return q


def _zipf_topk(T, d_in, k, rng):
    """Top-k sets whose channel frequencies fall off like 1 / (rank + 8): a few channels are
    nearly always selected, most rarely (the frequency imbalance the pages observe)."""
    p = 1.0 / (np.arange(d_in) + 8.0)
    p /= p.sum()
    perm = rng.permutation(d_in)
    return np.stack([perm[rng.choice(d_in, size=k, replace=False, p=p)] for _ in range(T)]).astype(np.int32)


def _ws(Q, T, n_dep):
    # filled with ones: the kernels must not depend on the scratch contents on entry
    return torch.full((max(Q.libqe.qe_cooccur_workspace_bytes(T, n_dep), 16),), 255, dtype=torch.uint8, device=DEV)


def _gpu_cooc(Q, topk, slot, n_dep, calls=1):
    t = torch.from_numpy(np.ascontiguousarray(topk)).to(DEV)
    s = torch.from_numpy(slot).to(DEV)
    cooc = torch.zeros(n_dep, n_dep, dtype=torch.int32, device=DEV)
    ws = _ws(Q, topk.shape[0], n_dep)
    for _ in range(calls):
        Q.libqe.qe_cooccur(t, s, n_dep, cooc, ws)
    torch.cuda.synchronize()
    return cooc.cpu().numpy().view(np.uint32).astype(np.int64)


@pytest.mark.parametrize("T,k,d_in,n_r,kind", [
    (1, 8, 64, 2, "zipf"),
    (255, 8, 256, 4, "zipf"),         # one ragged chunk
    (257, 16, 512, 4, "zipf"),        # a full chunk and one token
    (1000, 32, 4096, 8, "zipf"),      # the pages' k = 32, N_r = 8: 256 channels, 8 x 8 pair tiles
    (700, 33, 2048, 4, "zipf"),       # k above one register batch; 132 channels: a ragged pair tile
    (300, 100, 4096, 8, "zipf"),      # 800 channels
    (2000, 1, 512, 16, "zipf"),       # k = 1: only diagonal counts
    (128, 128, 8192, 8, "zipf"),      # 1024 channels: one full mask range
    (200, 64, 8192, 20, "zipf"),      # 1280 channels: two mask ranges, the second ragged
    (3000, 32, 4096, 8, "planted"),
])
def test_cooccur_bit_exact(Q, T, k, d_in, n_r, kind):
    rng = np.random.default_rng(T + k + d_in)
    if kind == "zipf":
        topk = _zipf_topk(T, d_in, k, rng)
    else:
        topk, _, _ = planted_topk(T, d_in, k, n_r, rng, cross_prob=0.1)
    hist = np.bincount(topk.reshape(-1), minlength=d_in)
    _, dep = C.frequency_partition(hist, k, n_r)
    indep, dep_lib, slot = Q.libqe.qe_partition_channels(hist.astype(np.uint32), k, n_r)
    np.testing.assert_array_equal(dep_lib, dep)
    got = _gpu_cooc(Q, topk, slot, len(dep))
    ref = C.cooccurrence(topk, dep, d_in)
    np.testing.assert_array_equal(got, ref)


def test_cooccur_accumulates_and_batches(Q):
    rng = np.random.default_rng(9)
    T, k, d_in, n_r = 1500, 32, 4096, 8
    topk = _zipf_topk(T, d_in, k, rng)
    hist = np.bincount(topk.reshape(-1), minlength=d_in)
    _, dep = C.frequency_partition(hist, k, n_r)
    _, _, slot = Q.libqe.qe_partition_channels(hist.astype(np.uint32), k, n_r)
    ref = C.cooccurrence(topk, dep, d_in)
    np.testing.assert_array_equal(_gpu_cooc(Q, topk, slot, len(dep), calls=2), 2 * ref)
    # the same tokens fed in two batches into one accumulator
    t = torch.from_numpy(topk).to(DEV)
    s = torch.from_numpy(slot).to(DEV)
    cooc = torch.zeros(len(dep), len(dep), dtype=torch.int32, device=DEV)
    ws = _ws(Q, T, len(dep))
    Q.libqe.qe_cooccur(t[:613], s, len(dep), cooc, ws)
    Q.libqe.qe_cooccur(t[613:], s, len(dep), cooc, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cooc.cpu().numpy().astype(np.int64), ref)


def test_cooccur_skips_out_of_range_entries(Q):
    rng = np.random.default_rng(10)
    T, k, d_in, n_r = 600, 16, 1024, 4
    topk = _zipf_topk(T, d_in, k, rng)
    hist = np.bincount(topk.reshape(-1), minlength=d_in)
    indep, dep = C.frequency_partition(hist, k, n_r)
    _, _, slot = Q.libqe.qe_partition_channels(hist.astype(np.uint32), k, n_r)
    bad = topk.copy()
    bad[::7, 3] = -1
    bad[::11, 5] = d_in + 5
    bad[::13, 0] = -(1 << 30)
    # the oracle's view: an out-of-range entry selects no token-dependent channel, the same
    # as an entry naming a token-independent one
    clean = bad.copy()
    clean[(clean < 0) | (clean >= d_in)] = indep[0]
    got = _gpu_cooc(Q, bad, slot, len(dep))
    np.testing.assert_array_equal(got, C.cooccurrence(clean, dep, d_in))


def test_cooccur_full_size_sampled(Q):
    # the calibration statistic of the 14336 -> 4096 down projection over 4096 tokens at
    # the pages' k = 32, N_r = 8; plus 65536 tokens, checked on the diagonal (the
    # histogram) and on sampled pairs counted one by one
    rng = np.random.default_rng(12)
    d_in, k, n_r = 14336, 32, 8
    for T in (4096, 65536):
        topk, _, _ = planted_topk(T, d_in, k, n_r, rng, cross_prob=0.2)
        hist = np.bincount(topk.reshape(-1), minlength=d_in)
        _, dep = C.frequency_partition(hist, k, n_r)
        _, _, slot = Q.libqe.qe_partition_channels(hist.astype(np.uint32), k, n_r)
        got = _gpu_cooc(Q, topk, slot, len(dep))
        if T == 4096:
            np.testing.assert_array_equal(got, C.cooccurrence(topk, dep, d_in))
            continue
        np.testing.assert_array_equal(np.diag(got), hist[dep])
        assert np.array_equal(got, got.T)
        O_occ = C.occurrence(topk, dep, d_in)
        for i, j in rng.integers(0, len(dep), (64, 2)):
            assert got[i, j] == int((O_occ[:, i] & O_occ[:, j]).sum())


def _planted_activations(T, d_in, k, n_groups, rng):
    """Activations whose top-k (with w = 1) holds k/2 of k 'always-on' channels and k/2
    channels of the token's group: a known answer for the whole calibration chain."""
    x = rng.normal(0.0, 0.3, (T, d_in)).astype(np.float32)
    chans = rng.permutation(d_in)
    always = chans[:k]
    groups = [chans[k + g * k: k + (g + 1) * k] for g in range(n_groups)]
    half = k // 2
    for t in range(T):
        g = rng.integers(n_groups)
        a = rng.choice(always, size=half, replace=False)
        b = rng.choice(groups[g], size=half, replace=False)
        x[t, a] = rng.uniform(5.0, 6.0, half) * rng.choice([-1.0, 1.0], half)
        x[t, b] = rng.uniform(3.0, 4.0, half) * rng.choice([-1.0, 1.0], half)
    return x, always, groups


def test_calibration_chain_recovers_planted_groups(Q):
    rng = np.random.default_rng(21)
    T, d_in, k, n_r = 2048, 4096, 32, 8
    x, always, groups = _planted_activations(T, d_in, k, n_r, rng)
    w = np.ones(d_in, np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    topk = torch.empty(T, k, dtype=torch.int32, device=DEV)
    hist = torch.zeros(d_in, dtype=torch.int32, device=DEV)
    Q.libqe.qe_channel_topk(xb.to(DEV), torch.from_numpy(w).to(DEV), k, topk, hist)
    torch.cuda.synchronize()
    t_ref, h_ref = O.channel_topk(xb.float().numpy(), w, k)
    assert np.array_equal(topk.cpu().numpy(), t_ref)
    h = hist.cpu().numpy().view(np.uint32)
    assert np.array_equal(h.astype(np.int64), h_ref)

    indep, dep, slot = Q.libqe.qe_partition_channels(h, k, n_r)
    o_indep, o_dep = C.frequency_partition(h_ref, k, n_r)
    assert np.array_equal(indep, o_indep) and np.array_equal(dep, o_dep)
    assert set(indep.tolist()) == set(always.tolist())

    cooc = torch.zeros(len(dep), len(dep), dtype=torch.int32, device=DEV)
    Q.libqe.qe_cooccur(topk, torch.from_numpy(slot).to(DEV), len(dep), cooc, _ws(Q, T, len(dep)))
    torch.cuda.synchronize()
    c = cooc.cpu().numpy().view(np.uint32)
    c_ref = C.cooccurrence(t_ref, o_dep, d_in)
    assert np.array_equal(c.astype(np.int64), c_ref)

    labels = Q.libqe.qe_cluster_channels(c, T, n_r, 0.2)
    o_labels, _, _, _ = C.cluster_channels(c_ref, T, n_r, 0.2)
    group_of = {int(ch): g for g, gs in enumerate(groups) for ch in gs}
    truth = C.canonical_labels(np.array([group_of[int(ch)] for ch in dep]))
    np.testing.assert_array_equal(labels, truth)
    np.testing.assert_array_equal(o_labels, truth)
