"""Exact int32 accumulators of the main product at the InternVL2-8B and Qwen2VL-72B widths.

For every linear of both layers (d_in up to 29568, d_out up to 29568; 128-token tiles and,
for the narrow k / v projections, 64-token tiles), in the benchmark's launch configuration:

  * the production prologue (qe_linear_prologue: route pass, route finish, expert-sorted
    quantization) writes codes and scales bit-identical to the oracle's for every token;
  * the main product with the accumulator dump (qe_wq_gemm with acc_debug) gives int32
    accumulators equal to the oracle's integer sums on sampled tokens (every column), so a
    lost or repeated 64-wide K step shows as a wrong integer;
  * the production epilogue (the same call without the dump, the fused fast path) writes
    y bit-identical to the dump path's y on every element, so the production output carries
    the checked accumulators.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import qe_oracle as O
from qe_testlib import f32

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [("internvl2_8b", l.name) for l in synth.get_config("internvl2_8b").linears]
CASES += [("qwen2vl_72b", l.name) for l in synth.get_config("qwen2vl_72b").linears]


@pytest.fixture(scope="module")
def Q():
    import quantized_linear_moe_amd as q
    return q


@pytest.fixture(scope="module")
def acts():
    cache = {}

    def get(cfg_name, stream):
        key = (cfg_name, stream)
        if key not in cache:
            cache.clear()
            cache[key] = synth.gen_activations(synth.get_config(cfg_name), stream)
        return cache[key]
    return get


@pytest.mark.parametrize("cfg_name,lin_name", CASES)
def test_accumulators_bit_exact_full_width(Q, acts, cfg_name, lin_name):
    cfg = synth.get_config(cfg_name)
    spec = next(l for l in cfg.linears if l.name == lin_name)
    params = synth.gen_linear(cfg, spec)
    layer = Q.QELinear.from_params(params, cfg.w_bits, cfg.a_bits, device=DEV)
    x = acts(cfg_name, spec.stream)
    T = x.shape[0]
    L = Q.libqe
    xd = x.to(DEV)
    ws = layer.workspace(T)
    codes = torch.empty(T, spec.d_in, dtype=torch.int8, device=DEV)
    s_x = torch.empty(T, dtype=torch.float32, device=DEV)
    u = torch.empty(T, L.rank_pad(cfg.r_shared), dtype=torch.bfloat16, device=DEV)
    v = torch.empty(T, L.rank_pad(cfg.r_routed), dtype=torch.bfloat16, device=DEV)
    e = torch.empty(T, dtype=torch.int32, device=DEV)
    perm = torch.empty(T, dtype=torch.int32, device=DEV)
    L.qe_linear_prologue(layer.lin, xd, codes, s_x, u, v, e, ws, perm=perm)
    y_dbg = torch.empty(T, spec.d_out, dtype=torch.float32, device=DEV)
    acc = torch.empty(T, spec.d_out, dtype=torch.int32, device=DEV)
    L.qe_wq_gemm(layer.lin, codes, s_x, None, T, u, v, e, y_dbg, acc, ws, perm=perm)
    y = torch.empty(T, spec.d_out, dtype=torch.float32, device=DEV)
    L.qe_wq_gemm(layer.lin, codes, s_x, None, T, u, v, e, y, None, ws, perm=perm)
    torch.cuda.synchronize()
    # production y carries the dumped accumulators: identical bits on every element
    same = torch.equal(y.view(torch.int32), y_dbg.view(torch.int32))
    assert same, f"fused epilogue differs from the dump path in {int((y != y_dbg).sum())} elements"
    # codes and scales of every token
    q_ref, sx_ref = O.quant_act(f32(x), params["s"], cfg.a_bits)
    assert np.array_equal(s_x.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(codes.cpu().numpy(), q_ref)
    # integer sums on sampled tokens (first and last always included), every column
    rng = np.random.default_rng(17)
    tok = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 48, replace=False)]))
    qw, _ = O.quant_weights(params["W_f"], params["s"], cfg.w_bits)
    acc_ref = q_ref[tok].astype(np.float64) @ qw.astype(np.float64).T
    got = acc[torch.as_tensor(tok, device=DEV)].cpu().numpy().astype(np.int64)
    bad = got != acc_ref.astype(np.int64)
    assert not bad.any(), f"{int(bad.sum())} accumulators differ (first at {np.argwhere(bad)[0].tolist()})"
