"""Linears that share one input (q/k/v, gate/up): qe_group_prologue / qe_group_forward.

The grouped route pass reads x once for all linears of the group and must give, bit for bit,
what each linear's own prologue and forward give (codes, scales, u, v, routes, bucketing and
y), on the grouped path (bf16 x, more than 16 tokens) and on the fallback path (float32 x,
few tokens), plus the oracle on sampled tokens of one linear.
"""

import numpy as np
import pytest
import torch

import synth
from qe_testlib import check_y, oracle_for

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def Q():
    import quantized_linear_moe_amd as q
    return q


def _layers(Q, cfg, names):
    specs = [next(l for l in cfg.linears if l.name == n) for n in names]
    params = [synth.gen_linear(cfg, sp) for sp in specs]
    layers = [Q.QELinear.from_params(p, cfg.w_bits, cfg.a_bits, device=DEV) for p in params]
    return specs, params, layers


# the grouped route pass, then the grouped route finish / expert-sorted pass / v finish (every
# linear routed with the same rank); ragged token counts (2000, 300: the few-token form)
CASES = [("qwen2vl_72b", ("q", "k", "v"), None), ("qwen2vl_72b", ("gate", "up"), None),
         ("qwen2vl_2b", ("q", "k", "v"), None), ("qwen2vl_2b", ("q", "k", "v"), 2000),
         ("internvl2_8b", ("gate", "up"), 300), ("tiny", ("lin",), None),
         ("qwen2vl_2b", ("q", "k", "v"), 200)]  # few tokens: each linear's one-launch prologue


@pytest.mark.parametrize("cfg_name,names,T", CASES)
def test_group_prologue_matches_single_prologues(Q, cfg_name, names, T):
    L = Q.libqe
    cfg = synth.get_config(cfg_name)
    specs, params, layers = _layers(Q, cfg, names)
    x = synth.gen_activations(cfg, specs[0].stream, T=T).to(DEV)
    T = x.shape[0]

    def bufs(spec):
        return dict(codes=torch.empty(T, spec.d_in, dtype=torch.int8, device=DEV),
                    s_x=torch.empty(T, device=DEV),
                    u=torch.empty(T, L.rank_pad(cfg.r_shared), dtype=torch.bfloat16, device=DEV),
                    v=torch.empty(T, L.rank_pad(cfg.r_routed), dtype=torch.bfloat16, device=DEV),
                    e=torch.empty(T, dtype=torch.int32, device=DEV), perm=torch.empty(T, dtype=torch.int32, device=DEV))
    single = [bufs(sp) for sp in specs]
    group = [bufs(sp) for sp in specs]
    for sp, lay, b in zip(specs, layers, single):
        L.qe_linear_prologue(lay.lin, x, b["codes"], b["s_x"], b["u"], b["v"], b["e"], lay.workspace(T),
                             perm=b["perm"])
    wss = [lay.workspace(T) for lay in layers]
    L.qe_group_prologue([l.lin for l in layers], x, [b["codes"] for b in group], [b["s_x"] for b in group],
                        [b["u"] for b in group], [b["v"] for b in group], [b["e"] for b in group], wss,
                        perm=[b["perm"] for b in group])
    torch.cuda.synchronize()
    for name, a, b in zip(names, single, group):
        for k in a:
            assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), f"{name}: {k} differs"


@pytest.mark.parametrize("cfg_name,names,T,dtype", [("qwen2vl_72b", ("q", "k", "v"), None, None),
                                                    ("qwen2vl_72b", ("gate", "up"), 1024, None),
                                                    ("internvl2_8b", ("q", "k", "v"), 12, None),
                                                    ("qwen2vl_2b", ("gate", "up"), 200, torch.float32),
                                                    ("internvl2_8b", ("q", "k", "v"), 160, None)])
def test_group_forward_matches_single_forwards(Q, cfg_name, names, T, dtype):
    L = Q.libqe
    cfg = synth.get_config(cfg_name)
    specs, params, layers = _layers(Q, cfg, names)
    x = synth.gen_activations(cfg, specs[0].stream, T=T)
    if dtype is not None:
        x = x.to(dtype)
    x = x.to(DEV)
    T = x.shape[0]
    ys1 = [torch.empty(T, sp.d_out, device=DEV) for sp in specs]
    es1 = [torch.empty(T, dtype=torch.int32, device=DEV) for _ in specs]
    for lay, y, e in zip(layers, ys1, es1):
        L.qe_linear_forward(lay.lin, x, y, e, lay.workspace(T))
    ys2 = [torch.full((T, sp.d_out), float("nan"), device=DEV) for sp in specs]
    es2 = [torch.full((T,), -1, dtype=torch.int32, device=DEV) for _ in specs]
    L.qe_group_forward([l.lin for l in layers], x, ys2, es2, [lay.workspace(T) for lay in layers])
    torch.cuda.synchronize()
    for name, a, b, ea, eb in zip(names, ys1, ys2, es1, es2):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{name}: y differs"
        assert torch.equal(ea, eb), f"{name}: routes differ"
    # and the oracle on sampled tokens of the last linear
    rng = np.random.default_rng(3)
    tok = np.unique(np.concatenate([[0, T - 1], rng.choice(T, min(T, 48), replace=False)]))
    xc = x.cpu()
    ref = oracle_for(params[-1], xc, cfg.w_bits, cfg.a_bits, tokens=tok)
    check_y(ys2[-1].cpu().numpy()[tok], ref, params[-1], xc[torch.as_tensor(tok)], cfg.w_bits, cfg.a_bits,
            gpu_expert=es2[-1].cpu().numpy()[tok])


def test_group_rejects_mismatched_inputs(Q):
    L = Q.libqe
    cfg = synth.get_config("qwen2vl_2b")
    specs, params, layers = _layers(Q, cfg, ("q", "down"))  # d_in 1536 and 8960
    x = synth.gen_activations(cfg, "x_attn").to(DEV)
    T = x.shape[0]
    ys = [torch.empty(T, sp.d_out, device=DEV) for sp in specs]
    with pytest.raises(L.QEError) as ex:
        L.qe_group_forward([l.lin for l in layers], x, ys, None, [lay.workspace(T) for lay in layers])
    assert ex.value.status == L.QE_ERR_INVALID_ARG


@pytest.mark.parametrize("cfg_name,names,T", [("qwen2vl_72b", ("q", "k", "v"), None), ("qwen2vl_72b", ("down",), None),
                                              ("qwen2vl_2b", ("q", "k", "v"), None), ("qwen2vl_2b", ("q", "k", "v"), 2000),
                                              ("qwen2vl_2b", ("q", "k", "v"), 300)])
def test_group_gemm_matches_single_gemms(Q, cfg_name, names, T):
    # one launch over the group's tiles against each linear's own launch: identical bits.  72B
    # q/k/v: 128-token tiles (the narrow k and v alone take 64-token tiles); 2B q/k/v at 2048
    # and 2000 tokens (a ragged last tile): 64-token tiles for the whole group (fewer than 512
    # 128-token tiles); at 300 tokens the K split keeps the per-linear launches
    L = Q.libqe
    cfg = synth.get_config(cfg_name)
    specs, params, layers = _layers(Q, cfg, names)
    x = synth.gen_activations(cfg, specs[0].stream, T=T).to(DEV)
    T = x.shape[0]
    wss = [lay.workspace(T) for lay in layers]
    bb = [dict(codes=torch.empty(T, sp.d_in, dtype=torch.int8, device=DEV), s_x=torch.empty(T, device=DEV),
               u=torch.empty(T, 32, dtype=torch.bfloat16, device=DEV), v=torch.empty(T, 32, dtype=torch.bfloat16, device=DEV),
               e=torch.empty(T, dtype=torch.int32, device=DEV), perm=torch.empty(T, dtype=torch.int32, device=DEV))
          for sp in specs]
    L.qe_group_prologue([l.lin for l in layers], x, [b["codes"] for b in bb], [b["s_x"] for b in bb],
                        [b["u"] for b in bb], [b["v"] for b in bb], [b["e"] for b in bb], wss,
                        perm=[b["perm"] for b in bb])
    ys1 = [torch.empty(T, sp.d_out, device=DEV) for sp in specs]
    for lay, b, y, w in zip(layers, bb, ys1, wss):
        L.qe_wq_gemm(lay.lin, b["codes"], b["s_x"], None, T, b["u"], b["v"], b["e"], y, None, w, perm=b["perm"])
    ys2 = [torch.full((T, sp.d_out), float("nan"), device=DEV) for sp in specs]
    L.qe_group_gemm([l.lin for l in layers], [b["codes"] for b in bb], [b["s_x"] for b in bb], T,
                    [b["u"] for b in bb], [b["v"] for b in bb], [b["e"] for b in bb], ys2, wss,
                    perm=[b["perm"] for b in bb])
    torch.cuda.synchronize()
    for name, a, b in zip(names, ys1, ys2):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{name}: y differs"
