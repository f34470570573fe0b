"""The allocation-free forward (qe_linear_forward_noalloc) against qe_linear_forward.

Both run the same kernels; the allocation-free call takes its workspace from the library's
per-GPU scratch array instead of a caller buffer, so outputs and routes must agree bit for
bit.  Each case makes two calls in a row, the second with fewer tokens (the array keeps the
first call's contents, which must not leak into the second).  A call whose workspace exceeds
the array is refused on the host before any launch.
"""

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def Q():
    import quantized_linear_moe_amd as q
    return q


CASES = [("tiny", "lin", 64, 37), ("qwen2vl_2b", "k", 300, 129), ("qwen2vl_72b_decode", "up", 8, 3),
         ("qwen2vl_72b_decode", "down", 16, 1)]


@pytest.mark.parametrize("cfg_name,lin_name,T1,T2", CASES)
def test_noalloc_forward_matches_forward(Q, cfg_name, lin_name, T1, T2):
    L = Q.libqe
    cfg = synth.get_config(cfg_name)
    spec = next(l for l in cfg.linears if l.name == lin_name)
    layer = Q.QELinear.from_params(synth.gen_linear(cfg, spec), cfg.w_bits, cfg.a_bits, device=DEV)
    x_all = synth.gen_activations(cfg, spec.stream, T=max(T1, T2)).to(DEV)
    assert L.qe_workspace_bytes(layer.lin, T1) <= L.qe_noalloc_scratch_bytes()
    for T in (T1, T2):
        x = x_all[:T].contiguous()
        y_ref = torch.empty(T, spec.d_out, dtype=torch.float32, device=DEV)
        e_ref = torch.empty(T, dtype=torch.int32, device=DEV)
        L.qe_linear_forward(layer.lin, x, y_ref, e_ref, layer.workspace(T))
        y = torch.full((T, spec.d_out), float("nan"), dtype=torch.float32, device=DEV)
        e = torch.full((T,), -1, dtype=torch.int32, device=DEV)
        L.qe_linear_forward_noalloc(layer.lin, x, y, e)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), f"T={T}: outputs differ"
        assert torch.equal(e, e_ref), f"T={T}: routes differ"


def test_noalloc_forward_refuses_oversized_call(Q):
    L = Q.libqe
    cfg = synth.get_config("qwen2vl_72b")
    spec = next(l for l in cfg.linears if l.name == "q")
    params = synth.gen_linear(cfg, spec, with_weight=False)
    params["W_f"] = np.zeros((spec.d_out, spec.d_in), np.float32)
    layer = Q.QELinear.from_params(params, cfg.w_bits, cfg.a_bits, device=DEV)
    T = 4096
    assert L.qe_workspace_bytes(layer.lin, T) > L.qe_noalloc_scratch_bytes()
    x = torch.zeros(T, spec.d_in, dtype=torch.bfloat16, device=DEV)
    y = torch.empty(T, spec.d_out, dtype=torch.float32, device=DEV)
    with pytest.raises(L.QEError) as ex:
        L.qe_linear_forward_noalloc(layer.lin, x, y, None)
    assert ex.value.status == L.QE_ERR_WORKSPACE
