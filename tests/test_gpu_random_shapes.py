"""GPU parity of the composite forward over seeded random shapes, against the oracle on sampled
tokens.  The cases are drawn so that every main-product path is met: 128-token tiles (the fast
epilogue, with the epilogue operands loaded in the K loop's last steps when there are at least
four K steps), 64-token tiles, K-split grids with their finish, the general epilogue (ranks above
32), tiles with more routed experts than one epilogue round holds, shared-only and routed-only
adapters, A6/A8, bf16 and float32 activations, ragged token and channel counts.  A second sweep
draws groups of linears that read one input (one launch over the group's tiles, the grouped
prologue when every linear is routed with one rank, the per-linear fallback otherwise): each
linear's y must match its own forward bit for bit and the oracle on sampled tokens.  A third sweep
draws few-token shapes (1 to 256 tokens, widths around the one-launch prologue's limit), checked on
every token."""

import numpy as np
import pytest
import torch

from qe_testlib import check_y, oracle_for

pytestmark = pytest.mark.gpu
DEV = "cuda"
N_TOK = 200  # sampled tokens per case for the oracle


@pytest.fixture(scope="module")
def Q():
    import quantized_linear_moe_amd as q
    return q


def _bf(a):
    return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)


def _params(rng, d_in, d_out, r_s, n_r, r_r):
    return dict(W_f=(rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32),
                s=rng.uniform(0.5, 2, d_in).astype(np.float32),
                A_s=_bf(rng.standard_normal((d_in, r_s)) * 0.02) if r_s else None,
                B_s=_bf(rng.standard_normal((r_s, d_out)) * 0.02) if r_s else None,
                A_r=_bf(rng.standard_normal((n_r, d_in, r_r)) * 0.02) if n_r else None,
                B_r=_bf(rng.standard_normal((n_r, r_r, d_out)) * 0.02) if n_r else None,
                R=_bf(rng.standard_normal((d_in, n_r)) * 0.02) if n_r else None)


def _x(rng, T, d_in, dtype):
    x = rng.standard_normal((T, d_in)).astype(np.float32)
    x[:, rng.choice(d_in, 2, replace=False)] *= 20.0  # always-on outlier channels
    return torch.from_numpy(x).to(dtype)


def _adapters(rng):
    r_s = int(rng.choice([0, 8, 32, 48]))
    n_r = int(rng.choice([0, 2, 8, 16])) if r_s else int(rng.choice([2, 8, 16]))
    r_r = int(rng.choice([8, 32, 64])) if n_r else 0
    return r_s, n_r, r_r


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    big = seed % 4 == 0  # enough 128-token tiles for the 128-token path
    T = int(rng.choice([4096, 4000, 3968])) if big else int(rng.integers(17, 1200))
    d_out = int(rng.choice([4096, 4112, 4352])) if big else int(rng.integers(1, 80)) * 16
    d_in = int(rng.choice([128, 256, 384, 640, 1024]))
    r_s, n_r, r_r = _adapters(rng)
    a_bits = int(rng.choice([6, 8]))
    x_dtype = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    return dict(T=T, d_in=d_in, d_out=d_out, r_s=r_s, n_r=n_r, r_r=r_r, a_bits=a_bits, x_dtype=x_dtype, rng=rng)


def _sample(rng, T):
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, min(T, N_TOK), replace=False)]))


@pytest.mark.parametrize("seed", range(20))
def test_random_shape_forward(Q, seed):
    c = _case(seed)
    rng = c["rng"]
    T, d_in, d_out, r_s, n_r, r_r = c["T"], c["d_in"], c["d_out"], c["r_s"], c["n_r"], c["r_r"]
    params = _params(rng, d_in, d_out, r_s, n_r, r_r)
    x = _x(rng, T, d_in, c["x_dtype"])
    print(f"seed {seed}: T {T} d_in {d_in} d_out {d_out} r_s {r_s} N_r {n_r} r_r {r_r} A{c['a_bits']} "
          f"{str(c['x_dtype']).split('.')[-1]}", flush=True)
    layer = Q.QELinear.from_params(params, 4, c["a_bits"], device=DEV)
    y = torch.full((T, d_out), float("nan"), dtype=torch.float32, device=DEV)
    e = torch.empty(T, dtype=torch.int32, device=DEV)
    Q.libqe.qe_linear_forward(layer.lin, x.to(DEV), y, e if n_r else None, layer.workspace(T))
    torch.cuda.synchronize()
    assert torch.isfinite(y).all(), "an output was not written"
    tok = _sample(rng, T)
    ref = oracle_for(params, x, 4, c["a_bits"], tokens=tok)
    err = check_y(y.cpu().numpy()[tok], ref, params, x[torch.as_tensor(tok)], 4, c["a_bits"],
                  gpu_expert=e.cpu().numpy()[tok] if n_r else None)
    print(f"  max rel err {err:.2e}")


def _group_case(seed):
    rng = np.random.default_rng(2000 + seed)
    n = int(rng.integers(2, 4))
    T = int(rng.choice([4096, 2048, 2000])) if seed % 2 == 0 else int(rng.integers(17, 700))
    d_in = int(rng.choice([256, 512, 1536]))
    d_outs = [int(rng.choice([512, 1024, 2048, 4096, 4112])) for _ in range(n)]
    if rng.random() < 0.6:  # every linear routed with one rank: the grouped prologue tails
        r_s, n_r, r_r = int(rng.choice([8, 32])), int(rng.choice([2, 8, 16])), int(rng.choice([8, 32]))
        ad = [(r_s, n_r, r_r)] * n
    else:
        ad = [_adapters(rng) for _ in range(n)]
    a_bits = int(rng.choice([6, 8]))
    x_dtype = torch.bfloat16 if rng.random() < 0.8 else torch.float32
    return dict(T=T, d_in=d_in, d_outs=d_outs, ad=ad, a_bits=a_bits, x_dtype=x_dtype, rng=rng)


@pytest.mark.parametrize("seed", range(10))
def test_random_group_forward(Q, seed):
    L = Q.libqe
    c = _group_case(seed)
    rng, T, d_in, a_bits = c["rng"], c["T"], c["d_in"], c["a_bits"]
    print(f"group seed {seed}: T {T} d_in {d_in} d_out {c['d_outs']} (r_s, N_r, r_r) {c['ad']} A{a_bits} "
          f"{str(c['x_dtype']).split('.')[-1]}", flush=True)
    params = [_params(rng, d_in, d_out, *ad) for d_out, ad in zip(c["d_outs"], c["ad"])]
    layers = [Q.QELinear.from_params(p, 4, a_bits, device=DEV) for p in params]
    x = _x(rng, T, d_in, c["x_dtype"])
    xd = x.to(DEV)
    routed = [ad[1] > 0 for ad in c["ad"]]
    ys1 = [torch.empty(T, d, device=DEV) for d in c["d_outs"]]
    es1 = [torch.full((T,), -1, dtype=torch.int32, device=DEV) for _ in layers]
    for lay, y, e, r in zip(layers, ys1, es1, routed):
        L.qe_linear_forward(lay.lin, xd, y, e if r else None, lay.workspace(T))
    ys2 = [torch.full((T, d), float("nan"), device=DEV) for d in c["d_outs"]]
    es2 = [torch.full((T,), -1, dtype=torch.int32, device=DEV) for _ in layers]
    L.qe_group_forward([l.lin for l in layers], xd, ys2, es2, [lay.workspace(T) for lay in layers])
    torch.cuda.synchronize()
    tok = _sample(rng, T)
    xs = x[torch.as_tensor(tok)]
    for i, (p, a, b, ea, eb, r) in enumerate(zip(params, ys1, ys2, es1, es2, routed)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"linear {i}: y differs from its own forward"
        if r:
            assert torch.equal(ea, eb), f"linear {i}: routes differ from its own forward"
        ref = oracle_for(p, x, 4, a_bits, tokens=tok)
        err = check_y(b.cpu().numpy()[tok], ref, p, xs, 4, a_bits, gpu_expert=eb.cpu().numpy()[tok] if r else None)
        print(f"  linear {i}: max rel err {err:.2e}")


def _few_case(seed):
    rng = np.random.default_rng(3000 + seed)
    # decode sizes, up to 128 tokens, 129 to 256 tokens in turn
    T = int(rng.integers(*((1, 17), (17, 129), (129, 257))[seed % 3]))
    d_in = int(rng.choice([128, 384, 1024, 2048, 3584, 4096, 8192, 8320]))
    d_out = int(rng.integers(1, 64)) * 16
    r_s, n_r, r_r = _adapters(rng)
    a_bits = int(rng.choice([6, 8]))
    return dict(T=T, d_in=d_in, d_out=d_out, r_s=r_s, n_r=n_r, r_r=r_r, a_bits=a_bits, rng=rng)


# few tokens: the one-launch prologue (up to 128 tokens, or 256 without a shared expert, d_in <= 8192), the
# two passes past those limits, and the fused decode at 16 tokens or fewer; bf16 x
@pytest.mark.parametrize("seed", range(24))
def test_random_few_token_forward(Q, seed):
    c = _few_case(seed)
    rng = c["rng"]
    T, d_in, d_out, r_s, n_r, r_r = c["T"], c["d_in"], c["d_out"], c["r_s"], c["n_r"], c["r_r"]
    print(f"few seed {seed}: T {T} d_in {d_in} d_out {d_out} r_s {r_s} N_r {n_r} r_r {r_r} A{c['a_bits']}", flush=True)
    params = _params(rng, d_in, d_out, r_s, n_r, r_r)
    x = _x(rng, T, d_in, torch.bfloat16)
    layer = Q.QELinear.from_params(params, 4, c["a_bits"], device=DEV)
    y = torch.full((T, d_out), float("nan"), dtype=torch.float32, device=DEV)
    e = torch.empty(T, dtype=torch.int32, device=DEV)
    Q.libqe.qe_linear_forward(layer.lin, x.to(DEV), y, e if n_r else None, layer.workspace(T))
    torch.cuda.synchronize()
    assert torch.isfinite(y).all(), "an output was not written"
    ref = oracle_for(params, x, 4, c["a_bits"])
    err = check_y(y.cpu().numpy(), ref, params, x, 4, c["a_bits"], gpu_expert=e.cpu().numpy() if n_r else None)
    print(f"  max rel err {err:.2e}")
