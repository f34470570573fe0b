"""The forward entry points captured in a HIP graph and replayed.

A serving loop captures the whole step once and replays it.  The forward path only launches
kernels (no allocation, copy, fill or synchronization inside), so a captured call must give,
on every replay, bit for bit what the same call gives eagerly: nothing of a result may come
from the state an earlier call left in the workspace or in the library's scratch array.  Each
case replays its graph several times; before each replay the outputs are poisoned, and after
it an eager call on other inputs (the token order reversed) overwrites the shared workspace.
Shapes cover each path: the one-launch few-token prologue with the split main product, the
two-pass prologue with the 128- and 64-token GEMM tiles, the grouped linears, weight-only
prefill and decode, and the allocation-free entry point.
"""

import dataclasses

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
REPLAYS = 4


@pytest.fixture(scope="module")
def Q():
    import quantized_linear_moe_amd as q
    return q


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _replay_and_check(g, outs, refs, perturb, label):
    for r in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else -7)
        g.replay()
        torch.cuda.synchronize()
        for k, (o, ref) in enumerate(zip(outs, refs)):
            assert torch.equal(_bits(o), _bits(ref)), f"{label}: replay {r}, output {k} differs from the eager call"
        perturb()
        torch.cuda.synchronize()


LINEAR_CASES = [
    ("tiny", "lin", None, None),               # few tokens: one-launch prologue, split-K main product
    ("qwen2vl_7b_s128", "up", None, None),     # Table 8 shape at 128 tokens
    ("qwen2vl_2b", "q", None, None),           # two-pass prologue, 64-token GEMM tiles
    ("qwen2vl_72b", "k", 1024, None),          # 128-token tiles, expert-sorted order
    ("qwen2vl_72b_decode", "up", None, None),  # W3A16 decode GEMV + finish
    ("internvl2_8b", "down", 600, (3, 16)),    # weight-only prefill (A16 GEMM)
    ("qwen2vl_72b_decode", "down", None, (4, 6)),  # quantized-activation decode
]


@pytest.mark.parametrize("cfg_name,lin_name,T,bits", LINEAR_CASES)
def test_linear_forward_graph_replays(Q, cfg_name, lin_name, T, bits):
    L = Q.libqe
    cfg = synth.get_config(cfg_name)
    if bits is not None:
        cfg = dataclasses.replace(cfg, w_bits=bits[0], a_bits=bits[1])
    spec = next(l for l in cfg.linears if l.name == lin_name)
    T = T or cfg.T
    layer = Q.QELinear.from_params(synth.gen_linear(cfg, spec), cfg.w_bits, cfg.a_bits, device=DEV)
    x = synth.gen_activations(cfg, spec.stream, T=T).to(DEV)
    x2 = x.flip(0).contiguous()
    ws = layer.workspace(T)
    y = torch.empty(T, spec.d_out, dtype=torch.float32, device=DEV)
    e = torch.empty(T, dtype=torch.int32, device=DEV)
    y2, e2 = torch.empty_like(y), torch.empty_like(e)
    fwd = lambda: L.qe_linear_forward(layer.lin, x, y, e, ws)
    fwd()
    torch.cuda.synchronize()
    refs = [y.clone(), e.clone()]
    g = _capture(fwd)
    _replay_and_check(g, [y, e], refs, lambda: L.qe_linear_forward(layer.lin, x2, y2, e2, ws),
                      f"{cfg_name}/{lin_name} T={T}")


@pytest.mark.parametrize("cfg_name,names,T", [("qwen2vl_2b", ("q", "k", "v"), None),
                                              ("qwen2vl_72b", ("gate", "up"), 512),
                                              ("internvl2_8b", ("q", "k", "v"), 200)])
def test_group_forward_graph_replays(Q, cfg_name, names, T):
    L = Q.libqe
    cfg = synth.get_config(cfg_name)
    specs = [next(l for l in cfg.linears if l.name == n) for n in names]
    layers = [Q.QELinear.from_params(synth.gen_linear(cfg, sp), cfg.w_bits, cfg.a_bits, device=DEV) for sp in specs]
    T = T or cfg.T
    x = synth.gen_activations(cfg, specs[0].stream, T=T).to(DEV)
    x2 = x.flip(0).contiguous()
    wss = [l.workspace(T) for l in layers]
    ys = [torch.empty(T, sp.d_out, dtype=torch.float32, device=DEV) for sp in specs]
    es = [torch.empty(T, dtype=torch.int32, device=DEV) for _ in specs]
    ys2, es2 = [torch.empty_like(y) for y in ys], [torch.empty_like(e) for e in es]
    lins = [l.lin for l in layers]
    fwd = lambda: L.qe_group_forward(lins, x, ys, es, wss)
    fwd()
    torch.cuda.synchronize()
    refs = [t.clone() for t in ys + es]
    g = _capture(fwd)
    _replay_and_check(g, ys + es, refs, lambda: L.qe_group_forward(lins, x2, ys2, es2, wss),
                      f"{cfg_name}/{'+'.join(names)} T={T}")


def test_noalloc_forward_graph_replays(Q):
    L = Q.libqe
    cfg = synth.get_config("qwen2vl_2b")
    spec = next(l for l in cfg.linears if l.name == "k")
    T = 300
    layer = Q.QELinear.from_params(synth.gen_linear(cfg, spec), cfg.w_bits, cfg.a_bits, device=DEV)
    assert L.qe_workspace_bytes(layer.lin, T) <= L.qe_noalloc_scratch_bytes()
    x = synth.gen_activations(cfg, spec.stream, T=T).to(DEV)
    x2 = x.flip(0).contiguous()
    y = torch.empty(T, spec.d_out, dtype=torch.float32, device=DEV)
    e = torch.empty(T, dtype=torch.int32, device=DEV)
    y2, e2 = torch.empty_like(y), torch.empty_like(e)
    fwd = lambda: L.qe_linear_forward_noalloc(layer.lin, x, y, e)
    fwd()
    torch.cuda.synchronize()
    # the eager forward with a caller workspace gives the same bits
    y_ws = torch.empty_like(y)
    e_ws = torch.empty_like(e)
    L.qe_linear_forward(layer.lin, x, y_ws, e_ws, layer.workspace(T))
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(y_ws)) and torch.equal(e, e_ws)
    refs = [y.clone(), e.clone()]
    g = _capture(fwd)
    _replay_and_check(g, [y, e], refs, lambda: L.qe_linear_forward_noalloc(layer.lin, x2, y2, e2),
                      f"noalloc qwen2vl_2b/k T={T}")
