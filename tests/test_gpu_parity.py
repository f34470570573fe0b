"""GPU parity: every libqe entry point against the CPU oracle on the same seeded inputs.

Bit-exact: activation codes and scales, int32 accumulators, routes (except router
near-ties, which are counted and accepted), bucketing, top-k sets/order and the
histogram.  Float outputs: max|y_gpu - y_ref| / max|y_ref| <= 2e-3 per linear.
Full-size configurations run the GPU in the benchmark's launch configuration and
compare sampled tokens (every output column of those tokens), which is exact
because every step is per-token.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import qe_oracle as O
from qe_testlib import check_routing, check_y, f32, near_ties, oracle_for, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def Q():
    import quantized_linear_moe_amd as q
    return q


def _layer(Q, cfg, spec, params=None, **override):
    params = params if params is not None else synth.gen_linear(cfg, spec)
    w_bits, a_bits = override.get("w_bits", cfg.w_bits), override.get("a_bits", cfg.a_bits)
    return Q.QELinear.from_params(params, w_bits, a_bits, device=DEV), params


def _spec(cfg, name):
    return next(l for l in cfg.linears if l.name == name)


def _codes_ref(x, s, a_bits):
    return O.quant_act(f32(x), s, a_bits)


# ------------------------------------------------------------------ a1 quant
@pytest.mark.parametrize("cfg_name,stream,lin_name", [("tiny", "x", "lin"), ("qwen2vl_2b", "x_attn", "q"),
                                                      ("qwen2vl_72b", "x_down", "down")])
def test_quant_act_bit_exact(Q, cfg_name, stream, lin_name):
    cfg = synth.get_config(cfg_name)
    x = synth.gen_activations(cfg, stream)
    s = synth.gen_linear(cfg, _spec(cfg, lin_name), with_weight=False)["s"]
    q_ref, sx_ref = _codes_ref(x, s, cfg.a_bits)
    xd = x.to(DEV)
    codes = torch.empty(x.shape, dtype=torch.int8, device=DEV)
    s_x = torch.empty(x.shape[0], dtype=torch.float32, device=DEV)
    Q.libqe.qe_quant_act(xd, torch.from_numpy(s).to(DEV), cfg.a_bits, codes, s_x)
    torch.cuda.synchronize()
    assert np.array_equal(s_x.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(codes.cpu().numpy(), q_ref)


def test_quant_act_golden_ties(Q):
    import json
    import os
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "rtn_act_cases.json")))["cases"]
    for c in cases:
        x = np.array(c["x"], np.float32)
        pad = (-x.shape[1]) % 8
        x = np.pad(x, ((0, 0), (0, pad)))
        s = None if c["s"] is None else np.pad(np.array(c["s"], np.float32), (0, pad), constant_values=1.0)
        codes = torch.empty(x.shape, dtype=torch.int8, device=DEV)
        s_x = torch.empty(x.shape[0], dtype=torch.float32, device=DEV)
        Q.libqe.qe_quant_act(torch.from_numpy(x).to(DEV), None if s is None else torch.from_numpy(s).to(DEV),
                             c["a_bits"], codes, s_x)
        torch.cuda.synchronize()
        got = codes.cpu().numpy()[:, :x.shape[1] - pad]
        assert got.tolist() == c["codes"], c["name"]
        assert s_x.cpu().numpy().tolist() == c["s_x"], c["name"]


# ------------------------------------------------------------------ a5 route
@pytest.mark.parametrize("cfg_name,lin_name", [("tiny", "lin"), ("qwen2vl_2b", "q"), ("qwen2vl_72b", "down")])
def test_route_parity(Q, cfg_name, lin_name):
    cfg = synth.get_config(cfg_name)
    spec = _spec(cfg, lin_name)
    params = synth.gen_linear(cfg, spec, with_weight=False)
    params["W_f"] = np.zeros((spec.d_out, spec.d_in), np.float32)  # weights do not enter routing
    layer, _ = _layer(Q, cfg, spec, params)
    x = synth.gen_activations(cfg, spec.stream)
    T, n_r = x.shape[0], cfg.n_routed
    ref = O.route(O.bf16_round(f32(x)) if x.dtype != torch.bfloat16 else f32(x), f32(params["R"]))
    i32 = dict(dtype=torch.int32, device=DEV)
    scores = torch.empty(T, n_r, dtype=torch.float32, device=DEV)
    expert, perm = torch.empty(T, **i32), torch.empty(T, **i32)
    counts, offsets = torch.empty(n_r, **i32), torch.empty(n_r + 1, **i32)
    Q.libqe.qe_route(layer.lin, x.to(DEV), scores, expert, counts, offsets, perm, layer.workspace(T))
    torch.cuda.synchronize()
    sc = scores.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(sc - ref["scores"])) <= 1e-5 * np.max(np.abs(ref["scores"]))
    e = expert.cpu().numpy()
    diff = check_routing(ref, e)
    print(f"near-ties: {int(near_ties(ref).sum())}, differing routes: {int(diff.sum())}")
    # bucketing is exact for the GPU's routes
    cnt = np.bincount(e, minlength=n_r)
    assert np.array_equal(counts.cpu().numpy(), cnt)
    assert np.array_equal(offsets.cpu().numpy(), np.concatenate([[0], np.cumsum(cnt)]))
    assert np.array_equal(perm.cpu().numpy(), np.argsort(e, kind="stable"))


# ------------------------------------------------------------ a3 accumulators
@pytest.mark.parametrize("cfg_name,lin_name,T,permute", [("tiny", "lin", None, False), ("tiny", "lin", 77, True),
                                                         ("qwen2vl_2b", "gate", None, False),
                                                         ("qwen2vl_2b", "k", 300, True), ("qwen2vl_2b", "q", 1000, True)])
def test_wq_gemm_acc_bit_exact(Q, cfg_name, lin_name, T, permute):
    cfg = synth.get_config(cfg_name)
    spec = _spec(cfg, lin_name)
    layer, params = _layer(Q, cfg, spec)
    x = synth.gen_activations(cfg, spec.stream, T=T)
    T = x.shape[0]
    xd = x.to(DEV)
    codes = torch.empty(x.shape, dtype=torch.int8, device=DEV)
    s_x = torch.empty(T, dtype=torch.float32, device=DEV)
    Q.libqe.qe_quant_act(xd, torch.from_numpy(params["s"]).to(DEV), cfg.a_bits, codes, s_x)
    y = torch.empty(T, spec.d_out, dtype=torch.float32, device=DEV)
    acc = torch.empty(T, spec.d_out, dtype=torch.int32, device=DEV)
    # the visiting order of the tokens must not change any result
    perm = torch.from_numpy(np.random.default_rng(T).permutation(T).astype(np.int32)).to(DEV) if permute else None
    Q.libqe.qe_wq_gemm(layer.lin, codes, s_x, None, T, None, None, None, y, acc, layer.workspace(T), perm=perm)
    torch.cuda.synchronize()
    qx, sx = _codes_ref(x, params["s"], cfg.a_bits)
    qw, s_w = O.quant_weights(params["W_f"], params["s"], cfg.w_bits)
    acc_ref, y_ref = O.main_term_int(qx, sx, qw, s_w)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), acc_ref)
    assert rel_err(y.cpu().numpy(), y_ref) <= 2e-3


# ------------------------------------------------------------ composite forward
FWD_CASES = [("tiny", "lin", None)]
FWD_CASES += [("qwen2vl_2b", l.name, None) for l in synth.get_config("qwen2vl_2b").linears]
FWD_CASES += [("internvl2_8b", n, 192) for n in ("q", "k", "gate", "down")]
FWD_CASES += [("qwen2vl_72b", l.name, 96) for l in synth.get_config("qwen2vl_72b").linears]


@pytest.mark.parametrize("cfg_name,lin_name,n_sample", FWD_CASES)
def test_linear_forward_parity(Q, cfg_name, lin_name, n_sample):
    cfg = synth.get_config(cfg_name)
    spec = _spec(cfg, lin_name)
    layer, params = _layer(Q, cfg, spec)
    x = synth.gen_activations(cfg, spec.stream)
    T = x.shape[0]
    y = torch.empty(T, spec.d_out, dtype=torch.float32, device=DEV)
    expert = torch.empty(T, dtype=torch.int32, device=DEV)
    layer.forward(x.to(DEV), y, expert)
    torch.cuda.synchronize()
    if n_sample is None:
        tokens = np.arange(T)
    else:  # sampled tokens, always including the first and the last (ragged) ones
        rng = np.random.default_rng(123)
        tokens = np.unique(np.concatenate([[0, T - 1], rng.choice(T, n_sample, replace=False)]))
    x_sub = x[torch.as_tensor(tokens)]
    ref = oracle_for(params, x, cfg.w_bits, cfg.a_bits, tokens=tokens)
    err = check_y(y.cpu().numpy()[tokens], ref, params, x_sub, cfg.w_bits, cfg.a_bits,
                  gpu_expert=expert.cpu().numpy()[tokens])
    print(f"{cfg_name}/{lin_name}: max rel err {err:.3e}, near-ties {int(near_ties(ref).sum())}")


# ------------------------------------------------------------ a7 decode (A16)
@pytest.mark.parametrize("lin_name", ["up", "down"])
def test_decode_w3a16_parity(Q, lin_name):
    cfg = synth.get_config("qwen2vl_72b_decode")
    spec = _spec(cfg, lin_name)
    layer, params = _layer(Q, cfg, spec)
    x = synth.gen_activations(cfg, spec.stream)
    y = torch.empty(x.shape[0], spec.d_out, dtype=torch.float32, device=DEV)
    expert = torch.empty(x.shape[0], dtype=torch.int32, device=DEV)
    layer.forward(x.to(DEV), y, expert)
    torch.cuda.synchronize()
    ref = oracle_for(params, x, cfg.w_bits, cfg.a_bits)
    err = check_y(y.cpu().numpy(), ref, params, x, cfg.w_bits, cfg.a_bits, gpu_expert=expert.cpu().numpy())
    print(f"decode {lin_name}: max rel err {err:.3e}")


@pytest.mark.parametrize("w_bits,T,x_dtype", [(4, 5, torch.bfloat16), (3, 16, torch.float32), (3, 37, torch.bfloat16)])
def test_decode_small_shapes(Q, w_bits, T, x_dtype):
    cfg = synth.get_config("tiny")
    spec = synth.LinearSpec("lin", 384, 272, "x")
    params = synth.gen_linear(cfg, spec)
    layer, _ = _layer(Q, cfg, spec, params, w_bits=w_bits, a_bits=16)
    x = (torch.randn(T, spec.d_in, generator=torch.Generator().manual_seed(w_bits * 100 + T)) * 3).to(x_dtype)
    y = torch.empty(T, spec.d_out, dtype=torch.float32, device=DEV)
    expert = torch.empty(T, dtype=torch.int32, device=DEV)
    layer.forward(x.to(DEV), y, expert)
    torch.cuda.synchronize()
    ref = oracle_for(params, x, w_bits, 16)
    check_y(y.cpu().numpy(), ref, params, x, w_bits, 16, gpu_expert=expert.cpu().numpy())


# weight-streaming GEMV: K ranges longer than the in-flight ring, workgroups whose waves get no
# K block, a partial last channel group, 16 tokens (smaller x tile budget) and the largest d_in
@pytest.mark.parametrize("w_bits,d_in,d_out,T", [(3, 4096, 1040, 8), (4, 3200, 400, 1), (3, 32768, 48, 2),
                                                 (4, 1152, 4096, 16), (3, 8192, 272, 13)])
def test_decode_stream_shapes(Q, w_bits, d_in, d_out, T):
    cfg = synth.get_config("tiny")
    spec = synth.LinearSpec("lin", d_in, d_out, "x")
    params = synth.gen_linear(cfg, spec)
    layer, _ = _layer(Q, cfg, spec, params, w_bits=w_bits, a_bits=16)
    x = (torch.randn(T, d_in, generator=torch.Generator().manual_seed(d_in + T)) * 2).to(torch.bfloat16)
    y = torch.empty(T, d_out, dtype=torch.float32, device=DEV)
    expert = torch.empty(T, dtype=torch.int32, device=DEV)
    layer.forward(x.to(DEV), y, expert)
    torch.cuda.synchronize()
    ref = oracle_for(params, x, w_bits, 16)
    err = check_y(y.cpu().numpy(), ref, params, x, w_bits, 16, gpu_expert=expert.cpu().numpy())
    print(f"stream W{w_bits} {d_in}x{d_out} T={T}: max rel err {err:.3e}")


# ------------------------------------------------------------ edge cases
def _custom(Q, d_in, d_out, T, w_bits=4, a_bits=8, r_s=8, n_r=4, r_r=8, seed=0, x_dtype=torch.bfloat16, x=None,
            R=None):
    rng = np.random.default_rng(seed)
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    params = dict(W_f=(rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32),
                  s=rng.uniform(0.5, 2, d_in).astype(np.float32) if a_bits != 16 else None,
                  A_s=bf(rng.standard_normal((d_in, r_s)) * 0.02) if r_s else None,
                  B_s=bf(rng.standard_normal((r_s, d_out)) * 0.02) if r_s else None,
                  A_r=bf(rng.standard_normal((n_r, d_in, r_r)) * 0.02) if n_r else None,
                  B_r=bf(rng.standard_normal((n_r, r_r, d_out)) * 0.02) if n_r else None,
                  R=(R if R is not None else bf(rng.standard_normal((d_in, n_r)) * 0.02)) if n_r else None)
    if x is None:
        x = torch.from_numpy(rng.standard_normal((T, d_in)).astype(np.float32) * 2).to(x_dtype)
    layer = Q.QELinear.from_params(params, w_bits, a_bits, device=DEV)
    y = torch.empty(T, d_out, dtype=torch.float32, device=DEV)
    expert = torch.empty(T, dtype=torch.int32, device=DEV)
    layer.forward(x.to(DEV), y, expert if n_r else None)
    torch.cuda.synchronize()
    ref = oracle_for(params, x, w_bits, a_bits)
    err = check_y(y.cpu().numpy(), ref, params, x, w_bits, a_bits, gpu_expert=expert.cpu().numpy() if n_r else None)
    return layer, params, x, y, expert, ref, err


@pytest.mark.parametrize("T", [1, 2, 129, 300])
def test_edge_token_counts(Q, T):
    _custom(Q, 256, 272, T, seed=T)


@pytest.mark.parametrize("a_bits,x_dtype", [(6, torch.float32), (8, torch.bfloat16), (6, torch.bfloat16)])
def test_edge_bits_and_dtypes(Q, a_bits, x_dtype):
    _custom(Q, 512, 400, 70, a_bits=a_bits, x_dtype=x_dtype, seed=a_bits)


def test_edge_rtn_and_shared_only(Q):
    _custom(Q, 256, 256, 50, r_s=0, n_r=0, r_r=0, seed=11)          # pure RTN baseline
    _custom(Q, 256, 256, 50, r_s=32, n_r=0, r_r=0, seed=12)         # shared expert only (LQER-style)
    _custom(Q, 256, 256, 50, r_s=0, n_r=3, r_r=16, seed=13)         # routed experts only
    _custom(Q, 256, 256, 50, r_s=64, n_r=16, r_r=48, seed=14)       # max experts, padded rank


def test_edge_all_tokens_one_expert_and_empty_experts(Q):
    rng = np.random.default_rng(5)
    d_in = 256
    x = torch.from_numpy(np.abs(rng.standard_normal((90, d_in))).astype(np.float32) + 0.1).to(torch.bfloat16)
    R = (rng.standard_normal((d_in, 4)) * 0.02).astype(np.float32)
    R[:, 2] = -1.0
    _, _, _, _, expert, ref, _ = _custom(Q, d_in, 512, 90, x=x, R=torch.from_numpy(R).to(torch.bfloat16), seed=5)
    assert np.all(expert.cpu().numpy() == 2)


def test_determinism_bitwise(Q):
    cfg = synth.get_config("qwen2vl_2b")
    spec = _spec(cfg, "down")
    layer, _ = _layer(Q, cfg, spec)
    x = synth.gen_activations(cfg, spec.stream).to(DEV)
    y1, y2 = layer.forward(x), layer.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


# ------------------------------------------------------------ a4/a6 pieces
def test_adapter_inputs_and_unfused_routed(Q):
    cfg = synth.get_config("qwen2vl_2b")
    spec = _spec(cfg, "o")
    layer, params = _layer(Q, cfg, spec)
    x = synth.gen_activations(cfg, spec.stream, T=500)
    T, d_out = x.shape[0], spec.d_out
    xd = x.to(DEV)
    ws = layer.workspace(T)
    i32 = dict(dtype=torch.int32, device=DEV)
    expert, perm = torch.empty(T, **i32), torch.empty(T, **i32)
    counts, offsets = torch.empty(cfg.n_routed, **i32), torch.empty(cfg.n_routed + 1, **i32)
    Q.libqe.qe_route(layer.lin, xd, None, expert, counts, offsets, perm, ws)
    u = torch.empty(T, cfg.r_shared, dtype=torch.bfloat16, device=DEV)
    v = torch.empty(T, cfg.r_routed, dtype=torch.bfloat16, device=DEV)
    Q.libqe.qe_adapter_inputs(layer.lin, xd, expert, u, v, ws)
    torch.cuda.synchronize()
    e = expert.cpu().numpy()
    xb = f32(x)
    u_ref = xb.astype(np.float64) @ f32(params["A_s"]).astype(np.float64)
    v_ref = np.stack([xb[t].astype(np.float64) @ f32(params["A_r"])[e[t]] for t in range(T)])
    assert rel_err(f32(u), u_ref) <= 8e-3 and rel_err(f32(v), v_ref) <= 8e-3
    # main product + shared expert, then the routed experts added by the grouped kernel
    codes = torch.empty(x.shape, dtype=torch.int8, device=DEV)
    s_x = torch.empty(T, dtype=torch.float32, device=DEV)
    Q.libqe.qe_quant_act(xd, torch.from_numpy(params["s"]).to(DEV), cfg.a_bits, codes, s_x)
    y = torch.empty(T, d_out, dtype=torch.float32, device=DEV)
    Q.libqe.qe_wq_gemm(layer.lin, codes, s_x, None, T, u, None, None, y, None, ws)
    Q.libqe.qe_routed_lora(layer.lin, xd, expert, offsets, perm, y, ws)
    torch.cuda.synchronize()
    ref = oracle_for(params, x, cfg.w_bits, cfg.a_bits)
    check_y(y.cpu().numpy(), ref, params, x, cfg.w_bits, cfg.a_bits, gpu_expert=e)


# ------------------------------------------------- a1/a4/a5/a6 fused prologue
def _check_prologue(Q, layer, params, x, a_bits, n_r, r_s, r_r):
    """qe_linear_prologue on x: codes and s_x bit-exact, routes exact except near-ties,
    perm the stable bucketing of the routes, u / v within bf16 rounding of the fp64 sums."""
    T, d_in = x.shape
    xd = x.to(DEV)
    i32 = dict(dtype=torch.int32, device=DEV)
    codes = torch.empty(T, d_in, dtype=torch.int8, device=DEV)
    s_x = torch.empty(T, dtype=torch.float32, device=DEV)
    u = torch.empty(T, Q.libqe.rank_pad(r_s), dtype=torch.bfloat16, device=DEV) if r_s else None
    v = torch.empty(T, Q.libqe.rank_pad(r_r), dtype=torch.bfloat16, device=DEV) if n_r else None
    expert = torch.empty(T, **i32) if n_r else None
    perm = torch.empty(T, **i32) if n_r else None
    ws = layer.workspace(T)
    Q.libqe.qe_linear_prologue(layer.lin, xd, codes, s_x, u, v, expert, ws, perm=perm)
    torch.cuda.synchronize()
    q_ref, sx_ref = O.quant_act(f32(x), params["s"], a_bits)
    assert np.array_equal(s_x.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(codes.cpu().numpy(), q_ref)
    xb = f32(x).astype(np.float64) if x.dtype == torch.bfloat16 else O.bf16_round(f32(x)).astype(np.float64)

    def close(got, want):
        err = np.abs(got.astype(np.float64) - want)
        assert np.all(err <= 2.0 ** -8 * np.abs(want) + 1e-3 * max(float(np.max(np.abs(want))), 1e-30))

    if r_s:
        close(f32(u)[:, :r_s], xb @ f32(params["A_s"]).astype(np.float64))
        assert not np.any(f32(u)[:, r_s:])
    if n_r:
        e = expert.cpu().numpy()
        check_routing(O.route(xb, f32(params["R"])), e)
        assert np.array_equal(perm.cpu().numpy(), np.argsort(e, kind="stable"))
        A_r = f32(params["A_r"]).astype(np.float64)
        v_ref = np.zeros((T, r_r))
        for j in range(n_r):
            idx = np.nonzero(e == j)[0]
            v_ref[idx] = xb[idx] @ A_r[j]
        close(f32(v)[:, :r_r], v_ref)
        assert not np.any(f32(v)[:, r_r:])


@pytest.mark.parametrize("cfg_name,lin_name", [("tiny", "lin"), ("qwen2vl_2b", "q"), ("qwen2vl_2b", "down"),
                                               ("internvl2_8b", "gate"), ("qwen2vl_72b", "down")])
def test_prologue_parity(Q, cfg_name, lin_name):
    cfg = synth.get_config(cfg_name)
    spec = _spec(cfg, lin_name)
    layer, params = _layer(Q, cfg, spec)
    x = synth.gen_activations(cfg, spec.stream)
    _check_prologue(Q, layer, params, x, cfg.a_bits, cfg.n_routed, cfg.r_shared, cfg.r_routed)


@pytest.mark.parametrize("T,r_s,n_r,r_r,x_dtype", [(17, 8, 4, 8, torch.bfloat16), (300, 8, 4, 8, torch.float32),
                                                   (129, 0, 0, 0, torch.bfloat16), (70, 32, 0, 0, torch.float32),
                                                   (50, 0, 3, 16, torch.bfloat16), (200, 64, 16, 48, torch.bfloat16)])
def test_prologue_shapes(Q, T, r_s, n_r, r_r, x_dtype):
    rng = np.random.default_rng(T)
    d_in, d_out = 384, 272
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    params = dict(W_f=(rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32),
                  s=rng.uniform(0.5, 2, d_in).astype(np.float32),
                  A_s=bf(rng.standard_normal((d_in, r_s)) * 0.02) if r_s else None,
                  B_s=bf(rng.standard_normal((r_s, d_out)) * 0.02) if r_s else None,
                  A_r=bf(rng.standard_normal((n_r, d_in, r_r)) * 0.02) if n_r else None,
                  B_r=bf(rng.standard_normal((n_r, r_r, d_out)) * 0.02) if n_r else None,
                  R=bf(rng.standard_normal((d_in, n_r)) * 0.02) if n_r else None)
    x = torch.from_numpy(rng.standard_normal((T, d_in)).astype(np.float32) * 2).to(x_dtype)
    layer = Q.QELinear.from_params(params, 4, 6, device=DEV)
    _check_prologue(Q, layer, params, x, 6, n_r, r_s, r_r)


# few-token prologue in one launch (bf16 x, d_in <= 8192, up to 128 tokens, or 256 without a shared
# expert): widths from one channel group to the limit, A6/A8, ranks up to 64; and just past the token and
# width limits, where the two passes take over
@pytest.mark.parametrize("T,d_in,a_bits,r_s,n_r,r_r", [(128, 3584, 6, 32, 8, 32), (128, 8192, 8, 32, 8, 32),
                                                       (33, 128, 8, 64, 16, 64), (97, 1024, 6, 0, 2, 8),
                                                       (256, 3584, 8, 0, 8, 32), (256, 640, 8, 8, 0, 0),
                                                       (129, 3584, 6, 32, 8, 32), (64, 8320, 6, 32, 8, 32)])
def test_prologue_few_tokens(Q, T, d_in, a_bits, r_s, n_r, r_r):
    rng = np.random.default_rng(T + d_in)
    d_out = 256
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    params = dict(W_f=(rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32),
                  s=rng.uniform(0.5, 2, d_in).astype(np.float32),
                  A_s=bf(rng.standard_normal((d_in, r_s)) * 0.02) if r_s else None,
                  B_s=bf(rng.standard_normal((r_s, d_out)) * 0.02) if r_s else None,
                  A_r=bf(rng.standard_normal((n_r, d_in, r_r)) * 0.02) if n_r else None,
                  B_r=bf(rng.standard_normal((n_r, r_r, d_out)) * 0.02) if n_r else None,
                  R=bf(rng.standard_normal((d_in, n_r)) * 0.02) if n_r else None)
    x = rng.standard_normal((T, d_in)).astype(np.float32) * 2
    x[:, rng.choice(d_in, 3, replace=False)] *= 25.0
    x = torch.from_numpy(x).to(torch.bfloat16)
    layer = Q.QELinear.from_params(params, 4, a_bits, device=DEV)
    _check_prologue(Q, layer, params, x, a_bits, n_r, r_s, r_r)


# ------------------------------------------------------------ a8 top-k
@pytest.mark.parametrize("cfg_name,lin_name", [("tiny", "lin"), ("internvl2_8b", "q"), ("internvl2_8b", "down")])
def test_channel_topk_bit_exact(Q, cfg_name, lin_name):
    cfg = synth.get_config(cfg_name)
    spec = _spec(cfg, lin_name)
    W = synth.gen_linear(cfg, spec)["W_f"]
    w = O.colmean_abs(W)
    x = synth.gen_activations(cfg, spec.stream)
    T, d = x.shape
    topk = torch.empty(T, cfg.k, dtype=torch.int32, device=DEV)
    hist = torch.zeros(d, dtype=torch.int32, device=DEV)
    xd, wd = x.to(DEV), torch.from_numpy(w).to(DEV)
    Q.libqe.qe_channel_topk(xd, wd, cfg.k, topk, hist)
    Q.libqe.qe_channel_topk(xd, wd, cfg.k, None, hist)  # the histogram accumulates
    torch.cuda.synchronize()
    t_ref, h_ref = O.channel_topk(f32(x), w, cfg.k)
    assert np.array_equal(topk.cpu().numpy(), t_ref)
    assert np.array_equal(hist.cpu().numpy().astype(np.int64), 2 * h_ref)


@pytest.mark.parametrize("k", [1, 5, 64, 256])
def test_channel_topk_ties_and_k(Q, k):
    rng = np.random.default_rng(k)
    x = np.round(rng.standard_normal((33, 256)) * 2).astype(np.float32)  # many exact ties
    x[4] = 0.0
    w = np.ones(256, np.float32)
    w[::7] = 0.5
    topk = torch.empty(33, k, dtype=torch.int32, device=DEV)
    hist = torch.zeros(256, dtype=torch.int32, device=DEV)
    Q.libqe.qe_channel_topk(torch.from_numpy(x).to(DEV), torch.from_numpy(w).to(DEV), k, topk, hist)
    torch.cuda.synchronize()
    t_ref, h_ref = O.channel_topk(x, w, k)
    assert np.array_equal(topk.cpu().numpy(), t_ref)
    assert np.array_equal(hist.cpu().numpy().astype(np.int64), h_ref)


# the threshold path and the exact path: mass ties that overflow the candidate list, k above
# the threshold path's limit, d_in not a multiple of 8 (scalar loads), the largest d_in, k = d_in,
# zero weights and -0 activations
@pytest.mark.parametrize("T,d_in,k,pattern,dtype", [
    (9, 14336, 32, "normal", torch.bfloat16),
    (5, 32768, 40, "normal", torch.float32),
    (7, 1001, 17, "normal", torch.float32),
    (6, 3000, 300, "normal", torch.bfloat16),
    (4, 5000, 32, "constant", torch.bfloat16),
    (5, 2048, 100, "few_levels", torch.float32),
    (3, 100, 100, "normal", torch.float32),
    (6, 4096, 1024, "few_levels", torch.bfloat16),
])
def test_channel_topk_paths(Q, T, d_in, k, pattern, dtype):
    rng = np.random.default_rng(d_in + k)
    if pattern == "normal":
        x = rng.standard_normal((T, d_in)).astype(np.float32)
    elif pattern == "constant":
        x = np.full((T, d_in), 1.5, np.float32)
    else:
        x = rng.integers(-3, 4, (T, d_in)).astype(np.float32)
    x[0, ::5] = -0.0
    x = torch.from_numpy(x).to(dtype)
    w = rng.uniform(0.5, 2.0, d_in).astype(np.float32)
    w[::11] = 0.0
    if pattern != "normal":
        w[:] = 1.0
    topk = torch.empty(T, k, dtype=torch.int32, device=DEV)
    hist = torch.zeros(d_in, dtype=torch.int32, device=DEV)
    Q.libqe.qe_channel_topk(x.to(DEV), torch.from_numpy(w).to(DEV), k, topk, hist)
    torch.cuda.synchronize()
    t_ref, h_ref = O.channel_topk(f32(x), w, k)
    assert np.array_equal(topk.cpu().numpy(), t_ref)
    assert np.array_equal(hist.cpu().numpy().astype(np.int64), h_ref)


def test_colmean_abs(Q):
    cfg = synth.get_config("qwen2vl_2b")
    W = synth.gen_linear(cfg, _spec(cfg, "gate"))["W_f"]
    Wb = torch.from_numpy(W).to(torch.bfloat16)
    w = torch.empty(W.shape[1], dtype=torch.float32, device=DEV)
    Q.libqe.qe_colmean_abs(Wb.to(DEV), w)
    torch.cuda.synchronize()
    ref = O.colmean_abs(f32(Wb))
    assert np.array_equal(w.cpu().numpy().view(np.uint32), ref.view(np.uint32))  # bf16 sums are exact in float64
    Q.libqe.qe_colmean_abs(torch.from_numpy(W).to(DEV), w)
    torch.cuda.synchronize()
    ref32 = O.colmean_abs(W)
    ulp = np.abs(w.cpu().numpy().view(np.int32).astype(np.int64) - ref32.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1
