"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, and rejects invalid layers before touching any device."""
import ctypes

import pytest
import torch

import mixture_experts_layer_38_amd as M


def _params(**kw):
    base = dict(dim=1024, n_routed=64, hidden=512, shared_hidden=1024, top_k=6, n_group=8, topk_group=3,
                score_fn="softmax", act="bf16", weight="bf16", max_tokens=4096)
    base.update(kw)
    return M.make_params(**base)


def test_library_exports_every_declared_function():
    lib = M.load_library()
    names = M.declared_functions()
    assert {"moe_cfg_create", "moe_layer_forward", "moe_router_forward", "moe_dispatch_forward",
            "moe_cfg_destroy", "moe_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    assert M.status_string(M.MOE_OK) == "ok"
    assert "invalid" in M.status_string(M.MOE_ERR_INVALID_ARG)
    assert "unsupported" in M.status_string(M.MOE_ERR_UNSUPPORTED)
    assert M.status_string(-99) == "unknown status"


@pytest.mark.parametrize("kw", [
    dict(n_routed=63),                       # E % G != 0
    dict(topk_group=9),                      # kg > G
    dict(top_k=25),                          # K > max
    dict(top_k=9, topk_group=1),             # K > kg * E / G (8 experts per group)
    dict(n_group=0),
    dict(dim=0),
    dict(max_tokens=-1),
    dict(score_fn=7),
    dict(out=2),                             # fp8 output
    dict(path=9),
    dict(act_quant=2),                       # no such activation quantisation
])
def test_invalid_layers_rejected(kw):
    st, h = M.create_cfg(_params(**kw))
    assert st == M.MOE_ERR_INVALID_ARG and not h.value


@pytest.mark.parametrize("kw", [
    dict(act="f32", weight="bf16"),          # mixed dtypes
    dict(act="bf16", weight="f32"),
    dict(dim=1000),                          # D % 32
    dict(hidden=500),                        # bf16 needs H % 128
    dict(shared_hidden=1000),
    dict(n_routed=1024, n_group=8),          # E > 512
    dict(max_tokens=400000, dim=7168),       # x rows past 32-bit byte offsets
    dict(max_tokens=1100000, hidden=2048),   # an expert's h rows past 32-bit byte offsets
    dict(act_quant=True),                    # e4m3 activations need e4m3 weights
    dict(act_quant=True, act="f32", weight="fp8"),
    dict(act_quant=True, weight="fp8", path="stream"),  # e4m3 activations run on the grouped kernels only
    dict(backward=True, weight="fp8"),       # the backward pass takes bf16 weights
    dict(backward=True, act="f32", weight="f32"),
])
def test_unsupported_layers_rejected(kw):
    st, h = M.create_cfg(_params(**kw))
    assert st == M.MOE_ERR_UNSUPPORTED and not h.value


def test_backward_flag_must_be_0_or_1():
    p = _params()
    p.backward = 2
    st, h = M.create_cfg(p)
    assert st == M.MOE_ERR_INVALID_ARG and not h.value


def test_null_arguments_rejected():
    lib = M.load_library()
    h = ctypes.c_void_p()
    assert lib.moe_cfg_create(None, ctypes.byref(h)) == M.MOE_ERR_INVALID_ARG
    p = _params()
    assert lib.moe_cfg_create(ctypes.byref(p), None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_forward(None, None, 0, None, None, None, None, None, None, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_router_forward(None, None, 0, None, None, None, None, None, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch_forward(None, None, 0, None, None, None, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_backward(None, None, 0, None, None, None, None, None, None, None, None, None,
                                  None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_cfg_destroy(None) == M.MOE_OK


def test_balance_entry_points_reject_bad_arguments():
    """Null pointers, E outside [1, 512] and a non-finite gamma are refused
    before anything is launched (host buffers stand in for device pointers)."""
    lib = M.load_library()
    counts = (ctypes.c_int32 * 8)()
    buf = (ctypes.c_float * 8)()
    c, b = ctypes.cast(counts, ctypes.c_void_p), ctypes.cast(buf, ctypes.c_void_p)
    bad = M.MOE_ERR_INVALID_ARG
    assert lib.moe_bias_update(None, 8, 0.01, b, None) == bad
    assert lib.moe_bias_update(c, 8, 0.01, None, None) == bad
    assert lib.moe_bias_update(c, 0, 0.01, b, None) == bad
    assert lib.moe_bias_update(c, 513, 0.01, b, None) == bad
    assert lib.moe_bias_update(c, 8, float("nan"), b, None) == bad
    assert lib.moe_bias_update(c, 8, float("inf"), b, None) == bad
    assert lib.moe_load_stats(None, 8, b, None) == bad
    assert lib.moe_load_stats(c, 8, None, None) == bad
    assert lib.moe_load_stats(c, 0, b, None) == bad
    assert lib.moe_load_stats(c, 600, b, None) == bad


def test_quantizer_entry_point_rejects_bad_arguments():
    """Sizes and null pointers are checked before anything is launched; an
    empty input launches nothing (host buffers stand in for device pointers)."""
    lib = M.load_library()
    buf = (ctypes.c_uint8 * 1024)()
    b = ctypes.cast(buf, ctypes.c_void_p)
    bad = M.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_e4m3_1x128(b, 2, 100, b, b, None) == bad      # cols % 128
    assert lib.moe_quantize_e4m3_1x128(b, 2, 0, b, b, None) == bad
    assert lib.moe_quantize_e4m3_1x128(b, -1, 128, b, b, None) == bad
    assert lib.moe_quantize_e4m3_1x128(b, 1 << 20, 1 << 15, b, b, None) == bad  # past 2^34 elements
    assert lib.moe_quantize_e4m3_1x128(None, 2, 128, b, b, None) == bad
    assert lib.moe_quantize_e4m3_1x128(b, 2, 128, None, b, None) == bad
    assert lib.moe_quantize_e4m3_1x128(b, 2, 128, b, None, None) == bad
    assert lib.moe_quantize_e4m3_1x128(None, 0, 128, None, None, None) == M.MOE_OK


def test_binding_tensor_check():
    """The binding's tensor check (CPU tensors stand in for device ones)."""
    from mixture_experts_layer_38_amd._binding import _check_tensor
    cpu = torch.device("cpu")
    t = torch.zeros((4, 8), dtype=torch.float32)
    _check_tensor("t", t, torch.float32, (4, 8), cpu)
    for args in ((t, torch.bfloat16, (4, 8)), (t, torch.float32, (4, 9)), (t.t(), torch.float32, (8, 4)),
                 (None, torch.float32, (4, 8)), (t.numpy(), torch.float32, (4, 8))):
        with pytest.raises(ValueError):
            _check_tensor("t", args[0], args[1], args[2], cpu)


def test_debug_build_exports_every_declared_function():
    """The bounds-checked debug library (built beside the release one) loads
    and exports the same functions; the release library's debug query says
    it is not a debug build."""
    import os
    from mixture_experts_layer_38_amd import _binding as B
    from mixture_experts_layer_38_amd import build as Bd
    assert os.path.exists(Bd.LIB_DEBUG), "run the build first (release and debug)"
    dbg = ctypes.CDLL(Bd.LIB_DEBUG)
    for n in M.declared_functions():
        assert hasattr(dbg, n), n
    lib = M.load_library()
    site, value = ctypes.c_int(7), ctypes.c_int(7)
    if B.LIB_PATH.endswith("libmoe_mi355x.so"):
        assert lib.moe_debug_status(ctypes.byref(site), ctypes.byref(value)) == M.MOE_ERR_UNSUPPORTED
        assert site.value == 0 and value.value == 0
    assert lib.moe_debug_status(None, ctypes.byref(value)) == M.MOE_ERR_INVALID_ARG
