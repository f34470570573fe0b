"""Pins for the oracle's QE linear: main term, shared/routed experts, router (CPU only).

Pins: pure-Python brute force on tiny inputs, the RTN special case (zero
adapters), full-rank recovery of x.W_f^T by the shared expert, routing
invariance when all routed experts are identical, and bucketing invariants.
"""

import numpy as np
import pytest

from oracle import qe_oracle as O


def _bf(a):
    return O.bf16_round(np.asarray(a, np.float32))


def _tiny(seed, T=7, d_in=32, d_out=24, r_s=4, n_r=3, r_r=4, a_bits=8):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d_in)).astype(np.float32)
    x[:, 2] *= 20
    s = rng.uniform(0.5, 2, d_in).astype(np.float32)
    W = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    p = dict(
        A_s=_bf(rng.standard_normal((d_in, r_s)) * 0.02), B_s=_bf(rng.standard_normal((r_s, d_out)) * 0.02),
        A_r=_bf(rng.standard_normal((n_r, d_in, r_r)) * 0.02), B_r=_bf(rng.standard_normal((n_r, r_r, d_out)) * 0.02),
        R=_bf(rng.standard_normal((d_in, n_r)) * 0.02),
    )
    return x, s, W, p


def test_main_term_brute_force_python_ints():
    x, s, W, _ = _tiny(0)
    qx, s_x = O.quant_act(x, s, 8)
    qw, s_w = O.quant_weights(W, s, 4)
    acc, y = O.main_term_int(qx, s_x, qw, s_w)
    for t in range(qx.shape[0]):
        for i in range(qw.shape[0]):
            ref = sum(int(qx[t, j]) * int(qw[i, j]) for j in range(qx.shape[1]))
            assert acc[t, i] == ref
            assert y[t, i] == ref * float(s_x[t]) * float(s_w[i])


def test_zero_adapters_reduce_to_rtn():
    # With no shared or routed expert, QE is the RTN baseline of the listing's tables:
    # y = (q_x s_x)(q_w s_w)^T, a textbook float64 product of the dequantized operands.
    x, s, W, _ = _tiny(1)
    qw, s_w = O.quant_weights(W, s, 4)
    out = O.qe_linear(x, False, s, qw, s_w, 8)
    qx, s_x = O.quant_act(x, s, 8)
    ref = (qx.astype(np.float64) * s_x[:, None]) @ (qw.astype(np.float64) * s_w[:, None]).T
    assert np.max(np.abs(out["y64"] - ref)) <= 1e-12 * np.max(np.abs(ref))
    d_in, d_out = x.shape[1], W.shape[0]
    zero = dict(A_s=np.zeros((d_in, 4), np.float32), B_s=np.zeros((4, d_out), np.float32),
                A_r=np.zeros((2, d_in, 4), np.float32), B_r=np.zeros((2, 4, d_out), np.float32),
                R=_bf(np.random.default_rng(9).standard_normal((d_in, 2))))
    out0 = O.qe_linear(x, False, s, qw, s_w, 8, **zero)
    assert np.array_equal(out0["y64"], out["y64"])


@pytest.mark.parametrize("w_bits", [3, 4])
def test_full_rank_shared_expert_recovers_fp_product(w_bits):
    # A_s = I and B_s = E^T with E = W_f - W_q (dequantized codes) make the shared
    # expert reconstruct the whole quantization error: with 16-bit activations the
    # QE output equals x.W_f^T (DeepRead "Method": the SE reconstructs E = W_f - W_q).
    rng = np.random.default_rng(2)
    T, d_in, d_out = 9, 64, 40
    x = _bf(rng.standard_normal((T, d_in)) * 3)
    W = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    qw, s_w = O.quant_weights(W, None, w_bits)
    Wq = qw.astype(np.float64) * s_w[:, None].astype(np.float64)
    E = W.astype(np.float64) - Wq
    out = O.qe_linear(x, True, None, qw, s_w, 16, A_s=np.eye(d_in), B_s=E.T)
    ref = x.astype(np.float64) @ W.astype(np.float64).T
    assert np.max(np.abs(out["y"] - ref)) <= 1e-5 * np.max(np.abs(ref))
    # without the adapter the error is the quantization error, far above 1e-5
    out_rtn = O.qe_linear(x, True, None, qw, s_w, 16)
    assert np.max(np.abs(out_rtn["y"] - ref)) > 1e-3 * np.max(np.abs(ref))


def test_router_brute_force_and_bucketing():
    x, s, W, p = _tiny(3, T=29, n_r=5)
    xb = _bf(x)
    r = O.route(xb, p["R"])
    for t in range(xb.shape[0]):
        scores = [sum(float(xb[t, j]) * float(p["R"][j, e]) for j in range(xb.shape[1])) for e in range(5)]
        best = min(range(5), key=lambda e: (scores[e], e))
        assert r["expert"][t] == best
    T = xb.shape[0]
    assert r["counts"].sum() == T and r["offsets"][0] == 0 and r["offsets"][-1] == T
    assert sorted(r["perm"].tolist()) == list(range(T))
    for e in range(5):
        seg = r["perm"][r["offsets"][e]:r["offsets"][e + 1]]
        assert np.all(r["expert"][seg] == e) and np.all(np.diff(seg) > 0)


def test_router_ties_and_special_cases():
    rng = np.random.default_rng(4)
    xb = _bf(np.abs(rng.standard_normal((11, 16))) + 0.1)
    R = _bf(rng.standard_normal((16, 4)) * 0.02)
    # two identical columns: the lower index wins
    R2 = R.copy()
    R2[:, 3] = R2[:, 1]
    e2 = O.route(xb, R2)["expert"]
    assert not np.any(e2 == 3)
    # one expert: everybody goes there
    assert np.all(O.route(xb, R[:, :1])["expert"] == 0)
    # a strongly negative column captures every (positive) token
    R3 = R.copy()
    R3[:, 2] = -1000.0
    assert np.all(O.route(xb, R3)["expert"] == 2)


def test_routed_term_brute_force_per_token():
    x, s, W, p = _tiny(5, T=13, n_r=4)
    xb = _bf(x)
    expert = O.route(xb, p["R"])["expert"]
    y = O.routed_term(xb, p["A_r"], p["B_r"], expert)
    for t in range(xb.shape[0]):
        e = expert[t]
        v = [sum(float(xb[t, j]) * float(p["A_r"][e, j, m]) for j in range(xb.shape[1])) for m in range(4)]
        ref = [sum(v[m] * float(p["B_r"][e, m, i]) for m in range(4)) for i in range(W.shape[0])]
        assert np.allclose(y[t], ref, rtol=1e-12, atol=1e-15)


def test_identical_experts_make_output_routing_invariant():
    x, s, W, p = _tiny(6, n_r=4)
    qw, s_w = O.quant_weights(W, s, 4)
    A_r = np.repeat(p["A_r"][:1], 4, axis=0)
    B_r = np.repeat(p["B_r"][:1], 4, axis=0)
    a = O.qe_linear(x, False, s, qw, s_w, 8, A_s=p["A_s"], B_s=p["B_s"], A_r=A_r, B_r=B_r, R=p["R"])
    R_other = _bf(np.random.default_rng(7).standard_normal(p["R"].shape))
    b = O.qe_linear(x, False, s, qw, s_w, 8, A_s=p["A_s"], B_s=p["B_s"], A_r=A_r, B_r=B_r, R=R_other)
    assert not np.array_equal(a["expert"], b["expert"])
    assert np.allclose(a["y64"], b["y64"], rtol=1e-12, atol=1e-12)
    # and it equals a shared expert of rank r_s + r_r made of both adapters
    xb = _bf(x)
    A = np.concatenate([p["A_s"], A_r[0]], axis=1)
    B = np.concatenate([p["B_s"], B_r[0]], axis=0)
    c = O.qe_linear(x, False, s, qw, s_w, 8, A_s=A, B_s=B)
    assert np.allclose(a["y64"], c["y64"], rtol=1e-10, atol=1e-12)
    assert xb.shape == x.shape


def test_adapters_read_bf16_of_unsmoothed_x():
    # The adapter input is x itself (rounded to bf16), not x/s: changing s changes
    # only the main term.
    x, s, W, p = _tiny(8)
    qw, s_w = O.quant_weights(W, s, 4)
    full = O.qe_linear(x, False, s, qw, s_w, 8, **p)
    base = O.qe_linear(x, False, s, qw, s_w, 8)
    xb = _bf(x).astype(np.float64)
    se = (xb @ p["A_s"]) @ p["B_s"]
    re = O.routed_term(_bf(x), p["A_r"], p["B_r"], full["expert"])
    assert np.allclose(full["y64"] - base["y64"], se + re, rtol=1e-9, atol=1e-12)


def test_route_top2_hand_example():
    # scores = x when R is the identity: row [3, 1, 2] -> experts 1 then 2; row [1, 1, 0] -> 2, then
    # the tie between 0 and 1 goes to the lower index 0; row [5, 5, 5] -> 0 then 1
    xb = np.array([[3.0, 1.0, 2.0], [1.0, 1.0, 0.0], [5.0, 5.0, 5.0]])
    r = O.route_top2(xb, np.eye(3))
    assert r["expert"].tolist() == [1, 2, 0] and r["expert2"].tolist() == [2, 0, 1]
    assert np.allclose(r["margin2"], [1.0, 0.0, 0.0])
    assert np.array_equal(r["expert"], O.route(xb, np.eye(3))["expert"])


def test_top2_with_two_experts_uses_both_for_every_token():
    # with N_r = 2 every token takes both routed experts, so the output is main + SE + RE_0 + RE_1
    # whatever the router says (R is random here)
    x, s, W, p = _tiny(40, n_r=2)
    qw, s_w = O.quant_weights(W, s, 4)
    out = O.qe_linear_top2(x, False, s, qw, s_w, 8, p["A_s"], p["B_s"], p["A_r"], p["B_r"], p["R"])
    xb = _bf(x)
    qx, s_x = O.quant_act(x, s, 8)
    _, y_main = O.main_term_int(qx, s_x, qw, s_w)
    want = y_main + O.lowrank(xb, p["A_s"], p["B_s"]) + O.lowrank(xb, p["A_r"][0], p["B_r"][0]) + \
        O.lowrank(xb, p["A_r"][1], p["B_r"][1])
    assert np.allclose(out["y64"], want, rtol=0, atol=1e-12)
    assert np.all(out["experts"][:, 0] != out["experts"][:, 1])
