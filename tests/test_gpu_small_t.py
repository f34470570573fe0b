"""GPU parity of the quantized linear at few tokens, where the main product splits its K
steps over workgroups (exact int32 partial sums added by a finish kernel): the listing's
Table 8 shapes (Qwen2VL-7B linears, prefill s = 128, W4A6 and W4A8) and decode with
quantized activations (Qwen2VL-72B MLP, T = 8)."""

import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import qe_oracle as O
from qe_testlib import check_y, oracle_for, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def Q():
    import quantized_linear_moe_amd as q
    return q


def _spec(cfg, name):
    return next(l for l in cfg.linears if l.name == name)


def _cfg(name, **kw):
    return dataclasses.replace(synth.get_config(name), **kw)


# main product alone: the split-K result equals the one-pass result bit for bit (the
# accumulator dump forces one pass), and both equal the oracle's exact accumulators
@pytest.mark.parametrize("cfg_name,lin_name,T", [("qwen2vl_7b_s128", "q", None), ("qwen2vl_7b_s128", "down", None),
                                                 ("qwen2vl_7b_s128", "up", 77), ("qwen2vl_72b_decode", "up", None),
                                                 ("qwen2vl_72b_decode", "down", 3)])
def test_split_k_main_product_bit_exact(Q, cfg_name, lin_name, T):
    cfg = _cfg(cfg_name, w_bits=4, a_bits=6)
    spec = _spec(cfg, lin_name)
    params = synth.gen_linear(cfg, spec)
    layer = Q.QELinear.from_params(params, 4, 6, device=DEV)
    x = synth.gen_activations(cfg, spec.stream, T=T)
    T = x.shape[0]
    codes = torch.empty(x.shape, dtype=torch.int8, device=DEV)
    s_x = torch.empty(T, dtype=torch.float32, device=DEV)
    Q.libqe.qe_quant_act(x.to(DEV), torch.from_numpy(params["s"]).to(DEV), 6, codes, s_x)
    ws = layer.workspace(T)
    y_split = torch.empty(T, spec.d_out, dtype=torch.float32, device=DEV)
    y_one = torch.empty_like(y_split)
    acc = torch.empty(T, spec.d_out, dtype=torch.int32, device=DEV)
    Q.libqe.qe_wq_gemm(layer.lin, codes, s_x, None, T, None, None, None, y_split, None, ws)
    Q.libqe.qe_wq_gemm(layer.lin, codes, s_x, None, T, None, None, None, y_one, acc, ws)
    torch.cuda.synchronize()
    assert np.array_equal(y_split.cpu().numpy().view(np.uint32), y_one.cpu().numpy().view(np.uint32))
    qx, sx = O.quant_act(x.float().numpy(), params["s"], 6)
    qw, s_w = O.quant_weights(params["W_f"], params["s"], 4)
    acc_ref, y_ref = O.main_term_int(qx, sx, qw, s_w)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), acc_ref)
    assert rel_err(y_split.cpu().numpy(), y_ref) <= 2e-3


# the whole QE linear (prologue, split-K main product, shared and routed terms)
@pytest.mark.parametrize("lin_name", ["q", "up", "down"])
@pytest.mark.parametrize("a_bits", [6, 8])
def test_table8_shapes_forward(Q, lin_name, a_bits):
    cfg = _cfg("qwen2vl_7b_s128", a_bits=a_bits)
    spec = _spec(cfg, lin_name)
    params = synth.gen_linear(cfg, spec)
    layer = Q.QELinear.from_params(params, 4, a_bits, device=DEV)
    x = synth.gen_activations(cfg, spec.stream)
    T = x.shape[0]
    y = torch.empty(T, spec.d_out, dtype=torch.float32, device=DEV)
    expert = torch.empty(T, dtype=torch.int32, device=DEV)
    layer.forward(x.to(DEV), y, expert)
    torch.cuda.synchronize()
    ref = oracle_for(params, x, 4, a_bits)
    err = check_y(y.cpu().numpy(), ref, params, x, 4, a_bits, gpu_expert=expert.cpu().numpy())
    print(f"7B {lin_name} W4A{a_bits} T={T}: max rel err {err:.3e}")


@pytest.mark.parametrize("lin_name", ["up", "down"])
@pytest.mark.parametrize("a_bits,T", [(6, 8), (8, 8), (6, 1), (8, 16)])
def test_decode_quantized_activations(Q, lin_name, a_bits, T):
    cfg = _cfg("qwen2vl_72b_decode", w_bits=4, a_bits=a_bits)
    spec = _spec(cfg, lin_name)
    params = synth.gen_linear(cfg, spec)
    layer = Q.QELinear.from_params(params, 4, a_bits, device=DEV)
    x = synth.gen_activations(cfg, spec.stream, T=T)
    y = torch.empty(T, spec.d_out, dtype=torch.float32, device=DEV)
    expert = torch.empty(T, dtype=torch.int32, device=DEV)
    layer.forward(x.to(DEV), y, expert)
    torch.cuda.synchronize()
    ref = oracle_for(params, x, 4, a_bits)
    err = check_y(y.cpu().numpy(), ref, params, x, 4, a_bits, gpu_expert=expert.cpu().numpy())
    print(f"decode {lin_name} W4A{a_bits} T={T}: max rel err {err:.3e}")


# decode with quantized activations runs the int8 weight-streaming path; without adapters its
# output is the dequantized exact accumulator, bit for bit the main GEMM's
@pytest.mark.parametrize("d_in,d_out,T,a_bits", [(8192, 29568, 8, 6), (29568, 8192, 3, 8), (1152, 4096, 16, 6),
                                                 (4096, 1040, 1, 8), (3200, 400, 5, 6)])
def test_decode_int8_main_term_bit_exact(Q, d_in, d_out, T, a_bits):
    rng = np.random.default_rng(d_in + T)
    params = dict(W_f=(rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32),
                  s=rng.uniform(0.5, 2, d_in).astype(np.float32))
    layer = Q.QELinear.from_params(params, 4, a_bits, device=DEV)
    x = torch.from_numpy((rng.standard_normal((T, d_in)) * 2).astype(np.float32)).to(torch.bfloat16)
    x[0, :7] = 40.0  # an outlier row segment
    xd = x.to(DEV)
    ws = layer.workspace(T)
    y_dec = torch.empty(T, d_out, dtype=torch.float32, device=DEV)
    layer.forward(xd, y_dec, None, ws)
    codes = torch.empty(T, d_in, dtype=torch.int8, device=DEV)
    s_x = torch.empty(T, dtype=torch.float32, device=DEV)
    Q.libqe.qe_quant_act(xd, torch.from_numpy(params["s"]).to(DEV), a_bits, codes, s_x)
    y_gemm = torch.empty_like(y_dec)
    Q.libqe.qe_wq_gemm(layer.lin, codes, s_x, None, T, None, None, None, y_gemm, None, ws)
    torch.cuda.synchronize()
    assert np.array_equal(y_dec.cpu().numpy().view(np.uint32), y_gemm.cpu().numpy().view(np.uint32))
    qx, sx = O.quant_act(x.float().numpy(), params["s"], a_bits)
    qw, s_w = O.quant_weights(params["W_f"], params["s"], 4)
    _, y_ref = O.main_term_int(qx, sx, qw, s_w)
    assert rel_err(y_dec.cpu().numpy(), y_ref) <= 2e-3


# weight-only (A16) linears with more than 16 tokens: the bf16-MFMA GEMM that uses every weight
# fragment for 64 or 128 tokens (ragged token tails, K splits, float32 activations)
A16_CASES = [(3, 3584, 3584, 128, torch.bfloat16), (3, 18944, 3584, 128, torch.bfloat16),
             (3, 3584, 18944, 128, torch.bfloat16), (4, 1152, 4096, 600, torch.bfloat16),
             (3, 4096, 1040, 17, torch.float32), (3, 8192, 272, 300, torch.bfloat16), (4, 256, 272, 1000, torch.float32)]
A16_CASES = [c + (32, 8, 32) for c in A16_CASES] + [
    (3, 4096, 1040, 700, torch.bfloat16, 64, 16, 64), (4, 2048, 528, 513, torch.bfloat16, 0, 3, 16),
    (3, 1024, 256, 2048, torch.bfloat16, 8, 0, 0)]


@pytest.mark.parametrize("w_bits,d_in,d_out,T,dtype,r_s,n_r,r_r", A16_CASES)
def test_a16_gemm_forward(Q, w_bits, d_in, d_out, T, dtype, r_s, n_r, r_r):
    # last cases: a ragged 256-channel tile with rank-64 adapters and 16 experts, routed experts
    # only, and a shared expert only
    rng = np.random.default_rng(d_in * 7 + T)
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    params = dict(W_f=(rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32), s=None,
                  A_s=bf(rng.standard_normal((d_in, r_s)) * 0.02) if r_s else None,
                  B_s=bf(rng.standard_normal((r_s, d_out)) * 0.02) if r_s else None,
                  A_r=bf(rng.standard_normal((n_r, d_in, r_r)) * 0.02) if n_r else None,
                  B_r=bf(rng.standard_normal((n_r, r_r, d_out)) * 0.02) if n_r else None,
                  R=bf(rng.standard_normal((d_in, n_r)) * 0.02) if n_r else None)
    layer = Q.QELinear.from_params(params, w_bits, 16, device=DEV)
    x = torch.from_numpy((rng.standard_normal((T, d_in)) * 2).astype(np.float32)).to(dtype)
    y = torch.empty(T, d_out, dtype=torch.float32, device=DEV)
    expert = torch.empty(T, dtype=torch.int32, device=DEV) if n_r else None
    layer.forward(x.to(DEV), y, expert)
    torch.cuda.synchronize()
    tokens = np.arange(T) if T <= 300 else np.unique(np.concatenate([[0, T - 1], rng.choice(T, 128, replace=False)]))
    x_sub = x[torch.as_tensor(tokens)]
    ref = oracle_for(params, x, w_bits, 16, tokens=tokens)
    err = check_y(y.cpu().numpy()[tokens], ref, params, x_sub, w_bits, 16,
                  gpu_expert=expert.cpu().numpy()[tokens] if n_r else None)
    print(f"A16 W{w_bits} {d_in}x{d_out} T={T}: max rel err {err:.3e}")


def test_a16_gemm_72b_prefill_sampled(Q):
    # Qwen2VL-72B up projection, W3A16, 4096 tokens: tokens sampled for the oracle
    cfg = _cfg("qwen2vl_72b_decode")
    spec = _spec(cfg, "up")
    params = synth.gen_linear(cfg, spec)
    layer = Q.QELinear.from_params(params, 3, 16, device=DEV)
    x = synth.gen_activations(synth.get_config("qwen2vl_72b"), "x_mlp")
    T = x.shape[0]
    y = torch.empty(T, spec.d_out, dtype=torch.float32, device=DEV)
    expert = torch.empty(T, dtype=torch.int32, device=DEV)
    layer.forward(x.to(DEV), y, expert)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    tokens = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 48, replace=False)]))
    x_sub = x[torch.as_tensor(tokens)]
    ref = oracle_for(params, x, 3, 16, tokens=tokens)
    err = check_y(y.cpu().numpy()[tokens], ref, params, x_sub, 3, 16, gpu_expert=expert.cpu().numpy()[tokens])
    print(f"72B up W3A16 T={T}: max rel err {err:.3e}")
