"""The bf16-output option (qe_linear.y_dtype = QE_BF16) on every path of qe_linear_forward and
qe_wq_gemm.

Bit-exact: the bf16 output is the round-to-nearest-even of the float32 output the same call
writes with y_dtype = QE_F32 (the oracle's pinned bf16_round applied to the GPU's float32 y).
Against the oracle: max|y_bf16 - y_ref| / max|y_ref| <= 2e-3 + 2^-9 (the float32 tolerance plus
one bf16 rounding of each element, at most 2^-9 of its magnitude).
"""

import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import qe_oracle as O
from qe_testlib import check_y, oracle_for

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL16 = 2e-3 + 2.0 ** -9


@pytest.fixture(scope="module")
def Q():
    import quantized_linear_moe_amd as q
    return q


# (config, linear, tokens, w_bits, a_bits): decode W3A16 / W4A6 (fused GEMV + finish), few-token
# W4A6 (K-split int8 product + finish), prefill W4A6 (64- and 128-token tiles, general epilogue),
# weight-only prefill (register-tile kernel, DMA-ring kernel), float32 x
CASES = [("qwen2vl_72b_decode", "up", 8, 3, 16), ("qwen2vl_72b_decode", "down", 8, 4, 6),
         ("qwen2vl_7b_s128", "q", 128, 4, 6), ("qwen2vl_2b", "q", None, 4, 6), ("internvl2_8b", "k", 700, 4, 8),
         ("qwen2vl_72b", "gate", 1024, 4, 6), ("qwen2vl_7b_s128", "up", 128, 3, 16), ("qwen2vl_2b", "down", 600, 3, 16),
         ("tiny", "lin", None, 4, 8)]


@pytest.mark.parametrize("cfg_name,lin_name,T,w_bits,a_bits", CASES)
def test_bf16_output_is_rounded_float32_output(Q, cfg_name, lin_name, T, w_bits, a_bits):
    cfg = dataclasses.replace(synth.get_config(cfg_name), w_bits=w_bits, a_bits=a_bits)
    spec = next(l for l in cfg.linears if l.name == lin_name)
    params = synth.gen_linear(cfg, spec)
    layer = Q.QELinear.from_params(params, w_bits, a_bits, device=DEV)
    x = synth.gen_activations(cfg, spec.stream, T=T)
    T = x.shape[0]
    xd = x.to(DEV)
    ws = layer.workspace(T)
    y32 = torch.empty(T, spec.d_out, dtype=torch.float32, device=DEV)
    e32 = torch.empty(T, dtype=torch.int32, device=DEV)
    Q.libqe.qe_linear_forward(layer.lin, xd, y32, e32, ws)
    layer.lin.y_dtype = Q.libqe.QE_BF16
    y16 = torch.empty(T, spec.d_out, dtype=torch.bfloat16, device=DEV)
    e16 = torch.empty(T, dtype=torch.int32, device=DEV)
    Q.libqe.qe_linear_forward(layer.lin, xd, y16, e16, ws)
    torch.cuda.synchronize()
    assert torch.equal(e16, e32)
    want = O.bf16_round(y32.cpu().numpy()).view(np.uint32) >> 16
    got = y16.cpu().view(torch.int16).numpy().astype(np.uint16).astype(np.uint32)
    bad = got != want
    assert not bad.any(), f"{int(bad.sum())} bf16 outputs are not the rounded float32 outputs"
    # against the oracle on sampled tokens
    rng = np.random.default_rng(5)
    tok = np.unique(np.concatenate([[0, T - 1], rng.choice(T, min(T, 64), replace=False)]))
    x_sub = x[torch.as_tensor(tok)]
    ref = oracle_for(params, x, w_bits, a_bits, tokens=tok)
    check_y(y16.float().cpu().numpy()[tok], ref, params, x_sub, w_bits, a_bits,
            gpu_expert=e16.cpu().numpy()[tok], tol=TOL16)


def test_bf16_output_wq_gemm_weight_streaming(Q):
    # qe_wq_gemm with a_bits 16 and few tokens: the weight-streaming kernel and its finish
    cfg = synth.get_config("qwen2vl_72b_decode")
    spec = next(l for l in cfg.linears if l.name == "down")
    layer = Q.QELinear.from_params(synth.gen_linear(cfg, spec, with_weight=True), 3, 16, device=DEV)
    x = synth.gen_activations(cfg, spec.stream).to(DEV)
    T = x.shape[0]
    ws = layer.workspace(T)
    L = Q.libqe
    y32 = torch.empty(T, spec.d_out, dtype=torch.float32, device=DEV)
    L.qe_wq_gemm(layer.lin, None, None, x, T, None, None, None, y32, None, ws)
    layer.lin.y_dtype = L.QE_BF16
    y16 = torch.empty(T, spec.d_out, dtype=torch.bfloat16, device=DEV)
    L.qe_wq_gemm(layer.lin, None, None, x, T, None, None, None, y16, None, ws)
    torch.cuda.synchronize()
    want = O.bf16_round(y32.cpu().numpy()).view(np.uint32) >> 16
    got = y16.cpu().view(torch.int16).numpy().astype(np.uint16).astype(np.uint32)
    assert np.array_equal(got, want)


def test_bf16_output_refused_where_y_is_added_to(Q):
    L = Q.libqe
    cfg = synth.get_config("tiny")
    spec = cfg.linears[0]
    layer = Q.QELinear.from_params(synth.gen_linear(cfg, spec), cfg.w_bits, cfg.a_bits, device=DEV)
    layer.lin.y_dtype = L.QE_BF16
    x = synth.gen_activations(cfg, spec.stream).to(DEV)
    T = x.shape[0]
    y = torch.zeros(T, spec.d_out, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(L.qe_top2_workspace_bytes(layer.lin, T), dtype=torch.uint8, device=DEV)
    with pytest.raises(L.QEError) as ex:
        L.qe_linear_forward_top2(layer.lin, x, y, None, None, ws)
    assert ex.value.status == L.QE_ERR_UNSUPPORTED
