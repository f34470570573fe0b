"""GPU parity of top-2 routing (qe_linear_forward_top2) against the oracle on every path of the
composite entry point: the general path (float32 activations), the two-pass prefill (A6, bf16),
the weight-only GEMM (more than 16 tokens), and the fused weight-streaming decode (W3A16 and
W4A6).  A GPU choice that differs from the oracle's is accepted when it is an equally valid
top-2 pair under the oracle's scores (near ties), and the output is then compared with the
oracle evaluated on the GPU's pair."""

import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import qe_oracle as O
from qe_testlib import NEAR_TIE_REL, Y_TOL, f32, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def Q():
    import quantized_linear_moe_amd as q
    return q


def _check(Q, params, x, w_bits, a_bits, tokens=None):
    layer = Q.QELinear.from_params(params, w_bits, a_bits, device=DEV)
    T = x.shape[0]
    d_out = params["W_f"].shape[0]
    y = torch.empty(T, d_out, dtype=torch.float32, device=DEV)
    e1 = torch.empty(T, dtype=torch.int32, device=DEV)
    e2 = torch.empty(T, dtype=torch.int32, device=DEV)
    ws = torch.empty(Q.libqe.qe_top2_workspace_bytes(layer.lin, T), dtype=torch.uint8, device=DEV)
    Q.libqe.qe_linear_forward_top2(layer.lin, x.to(DEV), y, e1, e2, ws)
    torch.cuda.synchronize()
    toks = np.arange(T) if tokens is None else tokens
    xs = x[torch.as_tensor(toks)]
    g = np.stack([e1.cpu().numpy()[toks], e2.cpu().numpy()[toks]], axis=1)
    s = params["s"] if a_bits != 16 else None
    qw, s_w = O.quant_weights(params["W_f"], s, w_bits)
    args = (f32(xs), xs.dtype == torch.bfloat16, s, qw, s_w, a_bits, f32(params.get("A_s")), f32(params.get("B_s")),
            f32(params.get("A_r")), f32(params.get("B_r")), f32(params.get("R")))
    ref = O.qe_linear_top2(*args)
    # the GPU's pair must be a valid top-2 choice under the oracle's scores
    sc = ref["scores"]
    srt = np.sort(sc, axis=1)
    tol = NEAR_TIE_REL * np.maximum(np.abs(sc).max(axis=1), 1e-30)
    rows = np.arange(len(toks))
    assert np.all(g[:, 0] != g[:, 1])
    assert np.all(sc[rows, g[:, 0]] <= srt[:, 0] + tol)
    assert np.all(sc[rows, g[:, 1]] <= srt[:, 1] + tol)
    same = np.all(g == ref["experts"], axis=1)
    if not np.all(same):
        ref = O.qe_linear_top2(*args, experts_override=g)
    err = rel_err(y.cpu().numpy()[toks], ref["y64"])
    assert err <= Y_TOL, err
    return err, float(np.mean(same))


def test_top2_general_path_fp32_tiny(Q):
    cfg = synth.get_config("tiny")
    spec = cfg.linears[0]
    params = synth.gen_linear(cfg, spec)
    x = synth.gen_activations(cfg, spec.stream)
    err, agree = _check(Q, params, x, cfg.w_bits, cfg.a_bits)
    print(f"tiny top-2: err {err:.2e}, pairs equal to the oracle's {agree:.3f}")


@pytest.mark.parametrize("lin_name", ["q", "down"])
def test_top2_two_pass_prefill_qwen2vl2b(Q, lin_name):
    cfg = synth.get_config("qwen2vl_2b")
    spec = next(l for l in cfg.linears if l.name == lin_name)
    params = synth.gen_linear(cfg, spec)
    x = synth.gen_activations(cfg, spec.stream)
    rng = np.random.default_rng(5)
    toks = np.unique(np.concatenate([[0, x.shape[0] - 1], rng.choice(x.shape[0], 200, replace=False)]))
    err, agree = _check(Q, params, x, cfg.w_bits, cfg.a_bits, tokens=toks)
    print(f"2B {lin_name} top-2: err {err:.2e}, pairs equal {agree:.3f}")


def test_top2_weight_only_gemm(Q):
    rng = np.random.default_rng(9)
    d_in, d_out, T, n_r = 2048, 784, 300, 8
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    params = dict(W_f=(rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32), s=None,
                  A_s=bf(rng.standard_normal((d_in, 32)) * 0.02), B_s=bf(rng.standard_normal((32, d_out)) * 0.02),
                  A_r=bf(rng.standard_normal((n_r, d_in, 32)) * 0.02),
                  B_r=bf(rng.standard_normal((n_r, 32, d_out)) * 0.02), R=bf(rng.standard_normal((d_in, n_r)) * 0.02))
    x = torch.from_numpy((rng.standard_normal((T, d_in)) * 2).astype(np.float32)).to(torch.bfloat16)
    err, agree = _check(Q, params, x, 3, 16)
    print(f"A16 top-2: err {err:.2e}, pairs equal {agree:.3f}")


@pytest.mark.parametrize("w_bits,a_bits", [(3, 16), (4, 6)])
def test_top2_decode(Q, w_bits, a_bits):
    cfg = dataclasses.replace(synth.get_config("qwen2vl_72b_decode"), w_bits=w_bits, a_bits=a_bits)
    spec = next(l for l in cfg.linears if l.name == "down")
    params = synth.gen_linear(cfg, spec)
    x = synth.gen_activations(cfg, spec.stream)
    err, agree = _check(Q, params, x, w_bits, a_bits)
    print(f"decode W{w_bits}A{a_bits} top-2: err {err:.2e}, pairs equal {agree:.3f}")


def test_top2_argument_errors(Q):
    cfg = synth.get_config("tiny")
    params = dict(synth.gen_linear(cfg, cfg.linears[0]))
    params["A_r"], params["B_r"], params["R"] = params["A_r"][:1], params["B_r"][:1], params["R"][:, :1]
    layer = Q.QELinear.from_params(params, cfg.w_bits, cfg.a_bits, device=DEV)  # one routed expert
    x = torch.zeros(4, cfg.linears[0].d_in, device=DEV)
    y = torch.empty(4, cfg.linears[0].d_out, device=DEV)
    assert Q.libqe.qe_top2_workspace_bytes(layer.lin, 4) == 0
    with pytest.raises(Q.libqe.QEError):
        Q.libqe.qe_linear_forward_top2(layer.lin, x, y, ws=torch.empty(1 << 20, dtype=torch.uint8, device=DEV))


@pytest.mark.parametrize("T,x_f32", [(4096, False), (4000, False), (4096, True)])
def test_top2_fused_epilogue_internvl2_8b_q(Q, T, x_f32):
    """128-token tiles on the fast epilogue without a K split take both routed corrections in the
    main product's epilogue (the tile grid of the 4096 x 4096 projection reaches 512 workgroups).
    Expert-sorted tiles meet many second experts, so the epilogue's further rounds run too; a
    ragged last tile (T = 4000), and float32 activations (general prologue) are covered."""
    cfg = synth.get_config("internvl2_8b")
    spec = next(l for l in cfg.linears if l.name == "q")
    params = synth.gen_linear(cfg, spec)
    x = synth.gen_activations(cfg, spec.stream)[:T]
    if x_f32:
        x = x.float()
    rng = np.random.default_rng(T + int(x_f32))
    toks = np.unique(np.concatenate([np.arange(0, 130), np.arange(T - 70, T), rng.choice(T, 150, replace=False)]))
    err, agree = _check(Q, params, x, cfg.w_bits, cfg.a_bits, tokens=toks)
    print(f"8B q top-2 (T {T}, float32 x {x_f32}): err {err:.2e}, pairs equal {agree:.3f}")


@pytest.mark.parametrize("r_s,n_r,r_r", [(0, 8, 32), (8, 16, 16), (32, 2, 32)])
def test_top2_fused_epilogue_adapter_layouts(Q, r_s, n_r, r_r):
    """The fused top-2 path over adapter layouts: no shared expert, the most experts (16, so
    the epilogue takes eight rounds of two) with a rank padded from 16 to 32, and two experts
    (every token takes both).  4096 tokens x 4096 channels: 512 tiles of 128 tokens."""
    rng = np.random.default_rng(11 + r_s + n_r)
    d_in, d_out, T = 1024, 4096, 4096
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    params = dict(W_f=(rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32),
                  s=rng.uniform(0.5, 2, d_in).astype(np.float32),
                  A_s=bf(rng.standard_normal((d_in, r_s)) * 0.02) if r_s else None,
                  B_s=bf(rng.standard_normal((r_s, d_out)) * 0.02) if r_s else None,
                  A_r=bf(rng.standard_normal((n_r, d_in, r_r)) * 0.02),
                  B_r=bf(rng.standard_normal((n_r, r_r, d_out)) * 0.02),
                  R=bf(rng.standard_normal((d_in, n_r)) * 0.02))
    x = torch.from_numpy((rng.standard_normal((T, d_in)) * 2).astype(np.float32)).to(torch.bfloat16)
    toks = np.unique(np.concatenate([np.arange(0, 64), np.arange(T - 64, T), rng.choice(T, 120, replace=False)]))
    err, agree = _check(Q, params, x, 4, 8, tokens=toks)
    print(f"top-2 fused r_s {r_s} N_r {n_r} r_r {r_r}: err {err:.2e}, pairs equal {agree:.3f}")
