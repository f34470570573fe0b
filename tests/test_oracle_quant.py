"""Pins for the oracle's rounding and quantization steps (CPU only).

Each test checks the oracle against something other than itself: torch's bf16
storage cast, hand-written expected codes, closed-form properties of
round-to-nearest quantization, and invariances that a wrong smoothing direction,
a wrong qmax or a wrong rounding rule would break.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import qe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(11)
    a = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(37.0),
        rng.standard_normal(1000).astype(np.float32) * np.float32(1e-30),
        np.array([0.0, -0.0, 1.0, 3.0e38, -3.0e38, 1e-40], np.float32),
    ])
    ref = torch.from_numpy(a).to(torch.bfloat16).float().numpy()
    got = O.bf16_round(a)
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1 + 2^-7: even mantissa (1.0) wins.
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: even mantissa (1 + 2^-6) wins.
    a = np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8)], np.float32)
    assert O.bf16_round(a).tolist() == [1.0, 1 + 2**-6, -1.0]


def _load_cases():
    with open(os.path.join(GOLDEN, "rtn_act_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _load_cases(), ids=lambda c: c["name"])
def test_quant_act_golden_cases(case):
    x = np.array(case["x"], np.float32)
    s = np.array(case["s"], np.float32) if case["s"] is not None else None
    q, s_x = O.quant_act(x, s, case["a_bits"])
    assert q.tolist() == case["codes"]
    assert s_x.tolist() == case["s_x"]


def _rand_acts(seed, T=37, d=96):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d)).astype(np.float32)
    x[:, 5] *= 25
    x[3] = 0.0  # an all-zero token
    s = rng.uniform(0.5, 2.0, d).astype(np.float32)
    return x, s


@pytest.mark.parametrize("a_bits", [6, 8])
def test_quant_act_rtn_properties(a_bits):
    x, s = _rand_acts(1)
    qmax = 2 ** (a_bits - 1) - 1
    q, s_x = O.quant_act(x, s, a_bits)
    xs = x.astype(np.float64) / s.astype(np.float64)
    nz = s_x > 0
    assert np.all(np.abs(q) <= qmax)
    # every non-zero token reaches the end of the range exactly once or more
    assert np.all(np.abs(q[nz]).max(axis=1) == qmax)
    assert np.all(q[~nz] == 0) and np.all(s_x[~nz] == 0)
    # round to nearest: |x'/s_x - q| <= 1/2 (up to float32 rounding of x' and the quotient)
    r = xs[nz] / s_x[nz, None].astype(np.float64)
    assert np.max(np.abs(r - q[nz])) <= 0.5 + 1e-5
    # and no other code in range is strictly nearer
    for delta in (-1, 1):
        alt = np.clip(q[nz].astype(np.int64) + delta, -qmax, qmax)
        assert np.all(np.abs(r - q[nz]) <= np.abs(r - alt) + 1e-6)
    # dequantization error bound of RTN
    assert np.all(np.abs(xs[nz] - q[nz] * s_x[nz, None]) <= 0.5 * s_x[nz, None] * (1 + 1e-5))


def test_quant_act_scale_and_smoothing_direction():
    x, s = _rand_acts(2)
    q, s_x = O.quant_act(x, s, 8)
    # scaling the tokens by a power of two leaves codes unchanged, scales s_x
    q2, s_x2 = O.quant_act(x * np.float32(8.0), s, 8)
    assert np.array_equal(q, q2) and np.array_equal(s_x2, s_x * np.float32(8.0))
    # smoothing divides: doubling every s_j halves s_x, codes unchanged
    q3, s_x3 = O.quant_act(x, s * np.float32(2.0), 8)
    assert np.array_equal(q, q3) and np.array_equal(s_x3, s_x / np.float32(2.0))
    # s = None is the identity
    q4, s_x4 = O.quant_act(x, None, 8)
    q5, s_x5 = O.quant_act(x, np.ones(x.shape[1], np.float32), 8)
    assert np.array_equal(q4, q5) and np.array_equal(s_x4, s_x5)


@pytest.mark.parametrize("w_bits", [3, 4])
def test_quant_weights_properties(w_bits):
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((40, 64)) * 0.02).astype(np.float32)
    W[7] = 0.0
    s = rng.uniform(0.5, 2.0, 64).astype(np.float32)
    qmax = {3: 3, 4: 7}[w_bits]
    q, s_w = O.quant_weights(W, s, w_bits)
    Wp = W.astype(np.float64) * s.astype(np.float64)
    nz = s_w > 0
    assert np.all(np.abs(q) <= qmax) and np.all(np.abs(q[nz]).max(axis=1) == qmax)
    assert np.all(q[7] == 0) and s_w[7] == 0
    r = Wp[nz] / s_w[nz, None]
    assert np.max(np.abs(r - q[nz])) <= 0.5 + 1e-5
    # weights are amplified by s: doubling s doubles s_w and keeps the codes
    q2, s_w2 = O.quant_weights(W, s * np.float32(2.0), w_bits)
    assert np.array_equal(q, q2) and np.array_equal(s_w2, s_w * np.float32(2.0))


def test_pack_w4_layout_and_roundtrip():
    # byte m holds code 2m in bits 0-3 and code 2m+1 in bits 4-7 (two's complement)
    codes = np.array([[3, -2, -7, 7, 0, -1]], np.int8)
    p = O.pack_w4(codes)
    assert p.tolist() == [[0xE3, 0x79, 0xF0]]
    rng = np.random.default_rng(4)
    c = rng.integers(-7, 8, (17, 64)).astype(np.int8)
    assert np.array_equal(O.unpack_w4(O.pack_w4(c)), c)


def test_pack_w3_layout_and_roundtrip():
    rng = np.random.default_rng(5)
    c = rng.integers(-3, 4, (5, 96)).astype(np.int8)
    p = O.pack_w3(c)
    assert p.shape == (5, 3, 3) and p.dtype == np.uint32
    # brute force with Python integers: code i of a group at bits 3i..3i+2 of a
    # 96-bit little-endian value split into three 32-bit words
    for r in range(5):
        for g in range(3):
            v = 0
            for i in range(32):
                v |= (int(c[r, g * 32 + i]) & 7) << (3 * i)
            words = [(v >> (32 * k)) & 0xFFFFFFFF for k in range(3)]
            assert [int(w) for w in p[r, g]] == words
    assert np.array_equal(O.unpack_w3(p), c)


def _load_weight_cases():
    with open(os.path.join(GOLDEN, "rtn_weight_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _load_weight_cases(), ids=lambda c: c["name"])
def test_quant_weights_golden_cases(case):
    # exact .5 ties must round to even (2.5 -> 2, 3.5 -> 4, 0.5 -> 0, 1.5 -> 2): a
    # floor(v + 0.5) or round-half-away quantizer fails these
    W = np.array(case["W"], np.float32)
    s = np.array(case["s"], np.float32) if case["s"] is not None else None
    q, s_w = O.quant_weights(W, s, case["w_bits"])
    assert q.tolist() == case["codes"]
    assert s_w.tolist() == case["s_w"]
