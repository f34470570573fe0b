"""C-ABI tests that need no GPU: the library loads, exports every declared entry
point, rejects bad arguments with the documented status before launching, and
its host-side weight packing and cost model agree with the oracle."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qe.h")


@pytest.fixture(scope="module")
def L():
    lib_path = os.path.join(ROOT, "quantized_linear_moe_amd", "libqe.so")
    if not os.path.exists(lib_path):  # a fresh checkout: build the HIP library (cross-compiles, no GPU needed)
        import importlib.util
        spec = importlib.util.spec_from_file_location("qe_build", os.path.join(ROOT, "quantized_linear_moe_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    from quantized_linear_moe_amd import _libqe
    return _libqe


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qe_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("qe_quant_act", "qe_route", "qe_wq_gemm", "qe_routed_lora", "qe_linear_forward", "qe_channel_topk",
              "qe_colmean_abs", "qe_prepare", "qe_pack_weights", "qe_linear_cost"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    lib = L.raw_library()
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(L.EXPORTED) == set(_declared_functions())
    assert L.qe_version().startswith("libqe")


def _lin(L, **kw):
    base = dict(d_in=256, d_out=512, w_bits=4, a_bits=8, r_shared=8, n_routed=4, r_routed=8)
    base.update(kw)
    return L.make_linear(**base)


def test_descriptor_validation(L):
    lib = L.raw_library()
    assert L.qe_prepared_bytes(_lin(L)) > 0
    for bad in (dict(w_bits=5), dict(a_bits=7), dict(n_routed=17), dict(r_shared=65), dict(d_in=0),
                dict(n_routed=2, r_routed=0), dict(n_routed=0, r_routed=8)):
        assert L.qe_prepared_bytes(_lin(L, **bad)) == 0, bad
    # unsupported but well formed: 3-bit weights with quantized activations, ragged shapes
    for uns in (dict(w_bits=3, a_bits=8), dict(d_in=200), dict(d_out=500)):
        lin = _lin(L, **uns)
        lin.prep = 4096
        st = lib.qe_linear_forward(ctypes.byref(lin), 4096, 1, 4, 8192, None, 8192, 1 << 30, None)
        assert st == L.QE_ERR_UNSUPPORTED, uns


def test_forward_argument_errors_before_launch(L):
    lib = L.raw_library()
    lin = _lin(L)
    lin.prep = None
    assert lib.qe_linear_forward(ctypes.byref(lin), 4096, 1, 4, 8192, None, 8192, 1 << 30, None) == L.QE_ERR_INVALID_ARG
    lin.prep = 4096 + 4  # misaligned
    assert lib.qe_linear_forward(ctypes.byref(lin), 4096, 1, 4, 8192, None, 8192, 1 << 30, None) == L.QE_ERR_ALIGNMENT
    lin.prep = 4096
    need = L.qe_workspace_bytes(lin, 64)
    assert need > 0
    assert lib.qe_linear_forward(ctypes.byref(lin), 4096, 1, 64, 8192, None, 8192, need - 1, None) == L.QE_ERR_WORKSPACE
    assert lib.qe_linear_forward(ctypes.byref(lin), 4096, 7, 64, 8192, None, 8192, need, None) == L.QE_ERR_INVALID_ARG
    assert lib.qe_linear_forward(ctypes.byref(lin), 4096 + 2, 1, 64, 8192, None, 8192, need, None) == L.QE_ERR_ALIGNMENT
    # T == 0 is a no-op that touches nothing
    assert lib.qe_linear_forward(ctypes.byref(lin), None, 1, 0, None, None, None, 0, None) == L.QE_OK
    assert lib.qe_linear_forward(ctypes.byref(lin), 4096, 1, -1, 8192, None, 8192, need, None) == L.QE_ERR_INVALID_ARG
    # router needs routed experts
    lin0 = _lin(L, n_routed=0, r_routed=0)
    lin0.prep = 4096
    ws0 = L.qe_workspace_bytes(lin0, 8)
    assert lib.qe_route(ctypes.byref(lin0), 4096, 1, 8, None, 8192, 8192, 8192, 8192, 8192, ws0, None) == L.QE_ERR_INVALID_ARG
    # a smoothing vector is rejected for weight-only (A16) layers
    lin16 = _lin(L, w_bits=3, a_bits=16)
    assert lib.qe_prepare(ctypes.byref(lin16), 4096, 4096, 4096, 4096, 4096, 4096, 4096, 4096, 8192, None) == \
        L.QE_ERR_INVALID_ARG


def test_step_argument_errors_before_launch(L):
    lib = L.raw_library()
    assert lib.qe_quant_act(4096, 1, None, 4, 256, 5, 8192, 8192, None) == L.QE_ERR_INVALID_ARG
    assert lib.qe_quant_act(4096, 1, None, 4, 252, 8, 8192, 8192, None) == L.QE_ERR_UNSUPPORTED
    assert lib.qe_quant_act(4097, 1, None, 4, 256, 8, 8192, 8192, None) == L.QE_ERR_ALIGNMENT
    assert lib.qe_quant_act(None, 1, None, 0, 256, 8, None, None, None) == L.QE_OK
    assert lib.qe_channel_topk(4096, 1, 8192, 4, 256, 257, None, 8192, None) == L.QE_ERR_INVALID_ARG
    assert lib.qe_channel_topk(4096, 1, 8192, 4, 4096, 2000, None, 8192, None) == L.QE_ERR_UNSUPPORTED
    assert lib.qe_channel_topk(4096, 1, 8192, 4, 65536, 8, None, 8192, None) == L.QE_ERR_UNSUPPORTED
    assert lib.qe_channel_topk(4096, 1, 8192, 4, 256, 0, None, 8192, None) == L.QE_ERR_INVALID_ARG
    assert lib.qe_colmean_abs(4096, 1, 0, 256, 8192, None) == L.QE_ERR_INVALID_ARG
    assert lib.qe_colmean_abs(4100, 1, 16, 256, 8192, None) == L.QE_ERR_ALIGNMENT
    assert L.qe_status_string(L.QE_ERR_WORKSPACE) == "QE_ERR_WORKSPACE"
    assert L.qe_last_hip_error() == 0


@pytest.mark.parametrize("w_bits,shape,smooth", [(4, (24, 64), True), (4, (40, 256), False), (3, (24, 96), False),
                                                  (3, (16, 256), False), (4, (1536, 1536), True)])
def test_pack_weights_matches_oracle(L, w_bits, shape, smooth):
    from oracle import qe_oracle as O
    rng = np.random.default_rng(sum(shape) + w_bits)
    W = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    W[3] = 0.0
    W[5, 7] = 0.3  # a row outlier
    s = rng.uniform(0.5, 2.0, shape[1]).astype(np.float32) if smooth else None
    packed, w_scale = L.qe_pack_weights(W, s, w_bits)
    qw, s_w = O.quant_weights(W, s, w_bits)
    assert np.array_equal(w_scale.view(np.uint32), s_w.view(np.uint32))
    ref = O.pack_w4(qw) if w_bits == 4 else O.pack_w3(qw)
    assert np.array_equal(packed, ref.reshape(-1).view(np.uint8))


def test_cost_matches_oracle_and_table7(L):
    from oracle import qe_oracle as O
    for (T, d_in, d_out, r_s, n_r, r_r) in [(64, 256, 512, 8, 4, 8), (4096, 8192, 29568, 32, 8, 32),
                                            (128, 3584, 3584, 32, 8, 32)]:
        lin = L.make_linear(d_in, d_out, 4, 6, r_s, n_r, r_r)
        im, am, _ = L.qe_linear_cost(lin, T, n_r, 2)
        c = O.linear_cost(T, d_in, d_out, r_s, n_r, r_r)
        assert im == c["int_macs"] and am == c["adapter_macs"]
    # Table 7 with r = 64 split evenly, N_r = 8, d = 3584, s = 128 (listing, Table 7)
    lin = L.make_linear(3584, 3584, 4, 6, 32, 8, 32)
    im, am, _ = L.qe_linear_cost(lin, 128, 8, 2)
    assert im + am == 128 * 3584 ** 2 + 128 * 3584 * (2 * 64 + 8)


@pytest.mark.parametrize("kw", [dict(r_shared=0, n_routed=0, r_routed=0), dict(r_shared=32, n_routed=0, r_routed=0),
                                dict(r_shared=0, n_routed=3, r_routed=16), dict(w_bits=3, a_bits=16),
                                dict(w_bits=4, a_bits=16, r_shared=64, n_routed=16, r_routed=48)])
@pytest.mark.parametrize("T", [0, 1, 7, 4096])
def test_buffer_sizes_for_every_configuration(L, kw, T):
    lin = _lin(L, **kw)
    assert L.qe_prepared_bytes(lin) > 0
    assert L.qe_workspace_bytes(lin, T) >= 0
    if T > 0:
        assert L.qe_workspace_bytes(lin, T) >= L.qe_workspace_bytes(lin, 1)


def test_y_dtype_field_is_validated():
    from quantized_linear_moe_amd import _libqe as L
    lin = L.make_linear(256, 512, 4, 8, 8, 4, 8)
    assert L.qe_workspace_bytes(lin, 64) > 0
    lin.y_dtype = L.QE_BF16
    assert L.qe_workspace_bytes(lin, 64) > 0
    lin.y_dtype = 2  # not a dtype
    assert L.qe_workspace_bytes(lin, 64) == 0
