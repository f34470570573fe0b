"""Pins for the oracle's channel-importance top-k, histogram, column mean and cost (CPU only)."""

import json
import math
import os

import numpy as np
import pytest

from oracle import qe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_topk(x, w, k):
    sc = np.abs(x.astype(np.float32)) * w.astype(np.float32)[None, :]
    out = []
    for t in range(x.shape[0]):
        order = sorted(range(x.shape[1]), key=lambda j: (-float(sc[t, j]), j))
        out.append(order[:k])
    return np.array(out, np.int64)


@pytest.mark.parametrize("k", [1, 4, 8, 31])
def test_topk_brute_force(k):
    rng = np.random.default_rng(k)
    x = rng.standard_normal((12, 31)).astype(np.float32)
    x[:, [3, 9]] *= 10
    w = rng.uniform(0.001, 0.05, 31).astype(np.float32)
    topk, hist = O.channel_topk(x, w, k)
    ref = _brute_topk(x, w, k)
    assert np.array_equal(topk, ref)
    assert np.array_equal(hist, np.bincount(ref.reshape(-1), minlength=31))


def test_topk_invariants():
    rng = np.random.default_rng(1)
    T, d, k = 20, 64, 8
    x = rng.standard_normal((T, d)).astype(np.float32)
    w = rng.uniform(0.001, 0.05, d).astype(np.float32)
    topk, hist = O.channel_topk(x, w, k)
    assert hist.sum() == T * k
    assert all(len(set(r)) == k for r in topk.tolist())
    # k = d selects every channel once per token
    _, hall = O.channel_topk(x, w, d)
    assert np.all(hall == T)
    # k = 1 is the argmax of |x|*w with the lowest index on ties
    t1, _ = O.channel_topk(x, w, 1)
    assert np.array_equal(t1[:, 0], np.argmax(np.abs(x) * w, axis=1))
    # w == 1: top-k of |x|
    t_ones, _ = O.channel_topk(x, np.ones(d, np.float32), k)
    assert np.array_equal(t_ones, _brute_topk(x, np.ones(d, np.float32), k))
    # scaling w by a power of two changes no set
    t_scaled, _ = O.channel_topk(x, w * np.float32(2.0 ** -5), k)
    assert np.array_equal(t_scaled, topk)
    # sign of x does not matter
    t_neg, _ = O.channel_topk(-x, w, k)
    assert np.array_equal(t_neg, topk)


def test_topk_tie_break_lower_index():
    x = np.array([[1.0, 2.0, 2.0, 1.0, 2.0, -2.0]], np.float32)
    w = np.ones(6, np.float32)
    topk, _ = O.channel_topk(x, w, 3)
    assert topk.tolist() == [[1, 2, 4]]
    topk, _ = O.channel_topk(x, w, 5)
    assert topk.tolist() == [[1, 2, 4, 5, 0]]
    x0 = np.zeros((1, 5), np.float32)
    topk, _ = O.channel_topk(x0, np.ones(5, np.float32), 2)
    assert topk.tolist() == [[0, 1]]


def test_colmean_abs_brute_force():
    rng = np.random.default_rng(2)
    W = (rng.standard_normal((13, 9)) * 0.02).astype(np.float32)
    w = O.colmean_abs(W)
    for j in range(9):
        ref = math.fsum(abs(float(W[i, j])) for i in range(13)) / 13
        assert w[j] == np.float32(ref)
    assert np.all(O.colmean_abs(np.full((4, 3), -0.5, np.float32)) == 0.5)


def test_cost_matches_table7_closed_form():
    # thelatestinai.com listing, Table 7: a d x d linear over s tokens costs
    # s*d^2 + s*d*(2r + N_r) multiply-adds and d^2 + r*d*(1 + N_r) parameters,
    # where r is the total rank split evenly between the shared and the routed
    # experts (DeepRead "Method": r = 64 split evenly, N_r = 8).
    with open(os.path.join(GOLDEN, "table7_complexity.json")) as f:
        g = json.load(f)
    for row in g["rows"]:
        d, s, r, n_r = row["d"], row["s"], row["r"], row["N_r"]
        c = O.linear_cost(s, d, d, r // 2, n_r, r // 2)
        assert c["int_macs"] == row["origin_compute"]
        assert c["int_macs"] + c["adapter_macs"] == row["qe_compute"]
        assert c["weight_params"] == row["origin_memory"]
        assert c["weight_params"] + c["adapter_params"] == row["qe_memory"]
