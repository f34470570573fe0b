"""The plain C oracle (oracle/qe_ref.c) against the numpy oracle and against the pins (CPU only).

The two oracles are written separately (straight C loops in index order; numpy array
operations with BLAS products) and share no code.  Integer results (codes, accumulators,
routes away from near-ties, bucketing, top-k lists and counts) must agree bit for bit,
float32 scales bit for bit, and float64 outputs to a few ulps of the summation order.
The C oracle also meets the hand-derived golden cases and brute-force pins directly.
"""

import json
import os

import numpy as np
import pytest

from oracle import qe_oracle as O
from oracle import qe_ref as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _built():
    if not os.path.exists(C.LIB):
        C.build()


def _bf(a):
    return O.bf16_round(np.asarray(a, np.float32))


def test_golden_activation_cases():
    with open(os.path.join(GOLDEN, "rtn_act_cases.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        x = np.array(case["x"], np.float32)
        s = np.array(case["s"], np.float32) if case["s"] is not None else None
        q, s_x = C.quant_act(x, s, case["a_bits"])
        assert q.tolist() == case["codes"], case["name"]
        assert s_x.tolist() == case["s_x"], case["name"]


def test_golden_weight_cases():
    with open(os.path.join(GOLDEN, "rtn_weight_cases.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        W = np.array(case["W"], np.float32)
        s = np.array(case["s"], np.float32) if case["s"] is not None else None
        q, s_w = C.quant_weights(W, s, case["w_bits"])
        assert q.tolist() == case["codes"], case["name"]
        assert s_w.tolist() == case["s_w"], case["name"]


@pytest.mark.parametrize("a_bits", [6, 8])
def test_quant_act_matches_numpy_oracle(a_bits):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((300, 1000)).astype(np.float32)
    x[:, 7] *= 30
    x[5] = 0
    s = rng.uniform(0.5, 2, 1000).astype(np.float32)
    q1, s1 = C.quant_act(x, s, a_bits)
    q2, s2 = O.quant_act(x, s, a_bits)
    assert np.array_equal(q1, q2)
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))


@pytest.mark.parametrize("w_bits", [3, 4])
def test_quant_weights_matches_numpy_oracle(w_bits):
    rng = np.random.default_rng(4)
    W = (rng.standard_normal((200, 768)) * 0.02).astype(np.float32)
    W[3] = 0
    s = rng.uniform(0.5, 2, 768).astype(np.float32)
    q1, s1 = C.quant_weights(W, s, w_bits)
    q2, s2 = O.quant_weights(W, s, w_bits)
    assert np.array_equal(q1, q2)
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))


def test_main_acc_brute_force_and_numpy():
    rng = np.random.default_rng(5)
    qx = rng.integers(-127, 128, (6, 40)).astype(np.int8)
    qw = rng.integers(-7, 8, (9, 40)).astype(np.int8)
    acc = C.main_acc(qx, qw)
    for t in range(6):
        for i in range(9):
            assert acc[t, i] == sum(int(qx[t, j]) * int(qw[i, j]) for j in range(40))
    qx = rng.integers(-127, 128, (64, 29568)).astype(np.int8)
    qw = rng.integers(-7, 8, (48, 29568)).astype(np.int8)
    acc_np = qx.astype(np.float64) @ qw.astype(np.float64).T
    assert np.array_equal(C.main_acc(qx, qw), acc_np.astype(np.int64))
    # the extreme of the 72B down projection: 127 * 7 * 29568 stays inside int32
    big = C.main_acc(np.full((1, 29568), 127, np.int8), np.full((1, 29568), 7, np.int8))
    assert big[0, 0] == 127 * 7 * 29568


def test_route_brute_force_ties_and_bucketing():
    # a hand-made score table: token 0 -> expert 2, token 1 ties between 0 and 1 -> 0,
    # token 2 -> expert 1; x is one-hot so the scores are rows of R
    R = np.array([[3.0, 1.0, -2.0], [0.5, 0.5, 4.0], [1.0, -1.0, 0.0]], np.float32)
    xb = np.eye(3, dtype=np.float32)
    r = C.route(xb, R)
    assert r["expert"].tolist() == [2, 0, 1]
    assert r["counts"].tolist() == [1, 1, 1]
    assert r["offsets"].tolist() == [0, 1, 2, 3]
    assert r["perm"].tolist() == [1, 2, 0]
    assert r["margin"].tolist() == [3.0, 0.0, 1.0]
    rng = np.random.default_rng(6)
    xb = _bf(rng.standard_normal((500, 256)))
    R = _bf(rng.standard_normal((256, 8)) * 0.02)
    r1, r2 = C.route(xb, R), O.route(xb, R)
    near = r2["margin"] < 1e-12 * np.maximum(r2["margin_scale"], 1e-300)
    assert np.array_equal(r1["expert"][~near], r2["expert"][~near])
    assert np.max(np.abs(r1["scores"] - r2["scores"])) <= 1e-13 * np.max(np.abs(r2["scores"]))
    e = r1["expert"]
    assert r1["counts"].sum() == 500 and r1["offsets"][-1] == 500
    assert np.array_equal(r1["perm"], np.argsort(e, kind="stable"))


@pytest.mark.parametrize("a_bits,w_bits,x_bf16", [(8, 4, False), (6, 4, True), (16, 3, True), (16, 4, False)])
def test_qe_linear_matches_numpy_oracle(a_bits, w_bits, x_bf16):
    rng = np.random.default_rng(7 + a_bits + w_bits)
    T, d_in, d_out, r_s, n_r, r_r = 70, 256, 96, 8, 4, 8
    x = rng.standard_normal((T, d_in)).astype(np.float32)
    x[:, 3] *= 20
    if x_bf16:
        x = _bf(x)
    s = rng.uniform(0.5, 2, d_in).astype(np.float32)
    W = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    p = dict(A_s=_bf(rng.standard_normal((d_in, r_s)) * 0.02), B_s=_bf(rng.standard_normal((r_s, d_out)) * 0.02),
             A_r=_bf(rng.standard_normal((n_r, d_in, r_r)) * 0.02),
             B_r=_bf(rng.standard_normal((n_r, r_r, d_out)) * 0.02), R=_bf(rng.standard_normal((d_in, n_r)) * 0.02))
    ss = s if a_bits != 16 else None
    qw, s_w = C.quant_weights(W, ss, w_bits)
    c = C.qe_linear(x, x_bf16, ss, qw, s_w, a_bits, want_acc=True, **p)
    n = O.qe_linear(x, x_bf16, ss, qw, s_w, a_bits, **p)
    if a_bits != 16:
        assert np.array_equal(c["codes"], n["codes"])
        assert np.array_equal(c["s_x"].view(np.uint32), n["s_x"].view(np.uint32))
        assert np.array_equal(c["acc"].astype(np.int64), n["acc"])
    near = n["margin"] < 1e-12 * n["margin_scale"]
    assert np.array_equal(c["expert"][~near], n["expert"][~near])
    assert np.max(np.abs(c["y64"] - n["y64"])) <= 1e-12 * np.max(np.abs(n["y64"]))


def test_qe_linear_thread_count_does_not_change_results():
    rng = np.random.default_rng(8)
    x = _bf(rng.standard_normal((33, 128)))
    s = rng.uniform(0.5, 2, 128).astype(np.float32)
    qw, s_w = C.quant_weights((rng.standard_normal((64, 128)) * 0.02).astype(np.float32), s, 4)
    A_s, B_s = _bf(rng.standard_normal((128, 8)) * 0.02), _bf(rng.standard_normal((8, 64)) * 0.02)
    n = C.num_threads()
    try:
        C.set_threads(1)
        a = C.qe_linear(x, True, s, qw, s_w, 6, A_s=A_s, B_s=B_s)["y64"]
        C.set_threads(max(n, 2))
        b = C.qe_linear(x, True, s, qw, s_w, 6, A_s=A_s, B_s=B_s)["y64"]
    finally:
        C.set_threads(n)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("k", [1, 8, 32, 200])
def test_channel_topk_matches_numpy_oracle(k):
    rng = np.random.default_rng(9 + k)
    x = rng.standard_normal((120, 700)).astype(np.float32)
    x[:, 11] *= 40
    x[7, :] = 0.0  # an all-zero token: every score ties, the lowest indices win
    x[8, ::3] = -0.0
    w = (rng.random(700) + 0.5).astype(np.float32)
    w[100:140] = w[99]  # equal weights
    t1, h1 = C.channel_topk(x, w, k)
    t2, h2 = O.channel_topk(x, w, k)
    assert np.array_equal(t1, t2)
    assert np.array_equal(h1, h2)
    assert t1[7].tolist() == list(range(k))
    assert h1.sum() == 120 * k


def test_colmean_abs_matches_numpy_oracle():
    rng = np.random.default_rng(10)
    W = (rng.standard_normal((300, 500)) * 0.02).astype(np.float32)
    a, b = C.colmean_abs(W), O.colmean_abs(W)
    assert np.max(np.abs(a.view(np.int32).astype(np.int64) - b.view(np.int32).astype(np.int64))) <= 1
