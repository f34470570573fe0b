"""GPU parity of the decode path (T <= 16: one launch streams the projection matrix and the packed
weights, one finish launch routes and adds the adapter terms) over every adapter layout the
finish takes: no adapters at all, shared only, routed only, the largest ranks and expert count at
16 tokens, quantized activations (int32 partials), a partial last channel group, long K
(many K splits per channel group), and outputs wide enough for the finish's 64-channel
workgroups."""

import numpy as np
import pytest
import torch

from qe_testlib import check_y, oracle_for

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def Q():
    import quantized_linear_moe_amd as q
    return q


def _params(d_in, d_out, r_s, n_r, r_r, a_bits, seed):
    rng = np.random.default_rng(seed)
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    return dict(W_f=(rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32),
                s=rng.uniform(0.5, 2, d_in).astype(np.float32) if a_bits != 16 else None,
                A_s=bf(rng.standard_normal((d_in, r_s)) * 0.02) if r_s else None,
                B_s=bf(rng.standard_normal((r_s, d_out)) * 0.02) if r_s else None,
                A_r=bf(rng.standard_normal((n_r, d_in, r_r)) * 0.02) if n_r else None,
                B_r=bf(rng.standard_normal((n_r, r_r, d_out)) * 0.02) if n_r else None,
                R=bf(rng.standard_normal((d_in, n_r)) * 0.02) if n_r else None)


CASES = [  # w_bits, a_bits, T, r_s, n_r, r_r, d_in, d_out
    (3, 16, 1, 0, 0, 0, 1024, 640),       # no projection workgroups: no routing to wait for
    (3, 16, 8, 32, 0, 0, 2048, 1040),     # shared expert only, partial last channel group
    (4, 16, 16, 0, 8, 32, 1024, 2048),    # routed experts only
    (4, 16, 16, 64, 16, 64, 1536, 4096),  # largest ranks and expert count, 16 tokens
    (4, 6, 5, 64, 16, 64, 1024, 784),     # quantized activations (int32 partials)
    (4, 8, 16, 8, 2, 8, 2048, 1024),
    (3, 16, 3, 8, 4, 8, 29568, 256),      # long K: many main K splits per channel group
    # outputs of 16384 channels and more: the finish's 64-channel workgroups (two token slots per
    # thread past 8 tokens, main partials past the four requested ahead, rank-64 register rows)
    (3, 16, 16, 32, 8, 32, 1024, 16384),
    (4, 16, 11, 64, 16, 64, 1024, 16400),  # ragged last channel group, rank 64
    (4, 6, 16, 32, 8, 32, 4096, 16384),    # int32 partials
    (3, 16, 13, 0, 8, 32, 4096, 18944),    # routed experts only
]


@pytest.mark.parametrize("w_bits,a_bits,T,r_s,n_r,r_r,d_in,d_out", CASES)
def test_decode_adapter_layouts(Q, w_bits, a_bits, T, r_s, n_r, r_r, d_in, d_out):
    params = _params(d_in, d_out, r_s, n_r, r_r, a_bits, seed=d_in + d_out + T)
    layer = Q.QELinear.from_params(params, w_bits, a_bits, device=DEV)
    g = torch.Generator().manual_seed(T * 7 + r_s)
    x = (torch.randn(T, d_in, generator=g) * 2).to(torch.bfloat16)
    y = torch.empty(T, d_out, dtype=torch.float32, device=DEV)
    expert = torch.empty(T, dtype=torch.int32, device=DEV)
    layer.forward(x.to(DEV), y, expert if n_r else None)
    torch.cuda.synchronize()
    ref = oracle_for(params, x, w_bits, a_bits)
    err = check_y(y.cpu().numpy(), ref, params, x, w_bits, a_bits, gpu_expert=expert.cpu().numpy() if n_r else None)
    print(f"decode W{w_bits}A{a_bits} T={T} r_s={r_s} n_r={n_r} r_r={r_r} {d_in}x{d_out}: max rel err {err:.3e}")
