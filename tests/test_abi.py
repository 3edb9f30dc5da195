"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
function include/nys_attn.h declares, and validates arguments before touching HIP."""
import ctypes
import os
import re

import pytest

from efficient_transformer_attention_segment_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nys_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nys_(?:attn|proj|flash)_\w+)\s*\(", text)))


def test_header_declares_the_api():
    names = declared_functions()
    assert {"nys_attn_create", "nys_attn_forward", "nys_attn_destroy",
            "nys_attn_forward_debug", "nys_attn_forward_varlen",
            "nys_attn_workspace_bytes", "nys_attn_last_error", "nys_proj_qkv",
            "nys_proj_out", "nys_attn_backward"} <= set(names)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(declared_functions()) == set(_lib.SIGNATURES)


def _create(*args):
    plan = ctypes.c_void_p(12345)
    st = _lib.lib().nys_attn_create(ctypes.byref(plan), *args)
    return st, plan.value


@pytest.mark.parametrize("args,status", [
    ((1, 1, 64, 32, 8, 33, 6, -1), _lib.NYS_E_ARG),          # bad dtype
    ((-1, 1, 64, 32, 8, 33, 6, 1), _lib.NYS_E_ARG),          # B < 0
    ((1, 1, 0, 32, 8, 33, 6, 1), _lib.NYS_E_ARG),            # n = 0
    ((1, 1, 64, 32, 0, 33, 6, 1), _lib.NYS_E_ARG),           # m = 0
    ((1, 1, 64, 32, 128, 33, 6, 1), _lib.NYS_E_ARG),         # m > n
    ((1, 1, 64, 32, 8, 32, 6, 1), _lib.NYS_E_ARG),           # even conv width
    ((1, 1, 64, 32, 8, 0, 6, 1), _lib.NYS_E_ARG),            # conv width 0
    ((1, 1, 64, 32, 8, 33, -1, 1), _lib.NYS_E_ARG),          # iterations < 0
    ((1, 1, 64, 32, 8, 33, 101, 1), _lib.NYS_E_ARG),         # iterations > 100
    ((1, 1, 64, 0, 8, 33, 6, 1), _lib.NYS_E_ARG),            # d = 0
    ((1, 1, 64, 48, 8, 33, 6, 1), _lib.NYS_E_UNSUPPORTED),   # d not built
    ((1, 1, 1024, 32, 512, 33, 6, 1), _lib.NYS_E_UNSUPPORTED),  # m > 256
    ((1, 1, 64, 32, 8, 67, 6, 1), _lib.NYS_E_UNSUPPORTED),   # conv width > 65
    ((1 << 12, 1 << 11, 64, 32, 8, 33, 6, 1), _lib.NYS_E_UNSUPPORTED),  # B*H = 2^23
])
def test_create_rejects_before_any_device_call(args, status):
    st, plan = _create(*args)
    assert st == status
    assert plan is None  # *plan set to NULL on failure
    assert _lib.nys_attn_last_error() != ""


def test_create_null_plan_pointer():
    assert _lib.lib().nys_attn_create(None, 1, 1, 64, 32, 8, 33, 6, 1) == _lib.NYS_E_ARG


def test_null_safe_entry_points():
    L = _lib.lib()
    L.nys_attn_destroy(None)
    assert L.nys_attn_workspace_bytes(None) == 0
    assert L.nys_attn_forward(None, None, None, None, None, None, None) == _lib.NYS_E_ARG
    assert L.nys_attn_forward_debug(None, None, None, None, None, None, None,
                                    None) == _lib.NYS_E_ARG
    assert L.nys_attn_forward_varlen(None, None, None, None, None, None, None, None,
                                     None) == _lib.NYS_E_ARG
    assert L.nys_attn_profile_enable(None, 4) == _lib.NYS_E_ARG
    assert L.nys_attn_backward(*([None] * 12)) == _lib.NYS_E_ARG
    n = ctypes.c_int(0)
    assert L.nys_attn_profile_read(None, None, 0, ctypes.byref(n)) == _lib.NYS_E_ARG


@pytest.mark.parametrize("args", [(1, 1, 64, 32, 8, 33, 6, 1),
                                  (1, 1, 60, 32, 8, 33, 6, 1)])  # m need not divide n
def test_valid_shape_without_gpu_reports_device(args):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, plan = _create(*args)
    assert st == _lib.NYS_E_DEVICE and plan is None
    assert "device" in _lib.nys_attn_last_error()


# Fake, 16-byte aligned, non-overlapping addresses: the projection entry points validate
# them on the host and never dereference them before the device check.
_X, _W, _Q, _K, _V = (0x10000000 * (i + 1) for i in range(5))


@pytest.mark.parametrize("dims,status", [
    ((0, 2, 64, 64, 128), _lib.NYS_E_ARG),           # B = 0
    ((1, 0, 64, 64, 128), _lib.NYS_E_ARG),           # H = 0
    ((1, 2, 0, 64, 128), _lib.NYS_E_ARG),            # n = 0
    ((1, 2, 64, 48, 128), _lib.NYS_E_UNSUPPORTED),   # d not built
    ((1, 2, 64, 64, 96), _lib.NYS_E_UNSUPPORTED),    # d_model not a multiple of 64
    ((1, 1, 64, 32, 128), _lib.NYS_E_UNSUPPORTED),   # H d = 32
    ((4096, 64, 4096, 128, 128), _lib.NYS_E_UNSUPPORTED),  # index range
])
def test_projections_reject_bad_shapes(dims, status):
    L = _lib.lib()
    assert L.nys_proj_qkv(_X, _W, _Q, _K, _V, *dims, None) == status
    assert L.nys_proj_out(_X, _W, _Q, *dims, None) == status
    assert _lib.nys_attn_last_error() != ""


def test_projections_reject_bad_pointers():
    L = _lib.lib()
    dims = (1, 2, 64, 64, 128)
    assert L.nys_proj_qkv(None, _W, _Q, _K, _V, *dims, None) == _lib.NYS_E_ARG
    assert L.nys_proj_qkv(_X, _W, _Q, _K, _V + 8, *dims, None) == _lib.NYS_E_ARG  # misaligned
    assert L.nys_proj_qkv(_X, _W, _X + 64, _K, _V, *dims, None) == _lib.NYS_E_ARG  # overlap
    assert L.nys_proj_out(_X, None, _Q, *dims, None) == _lib.NYS_E_ARG
    assert L.nys_proj_out(_X, _W, _W + 16, *dims, None) == _lib.NYS_E_ARG  # y overlaps w_o


def test_projections_valid_shape_without_gpu_reports_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    L = _lib.lib()
    dims = (2, 2, 100, 64, 192)  # ragged M and N tiles
    assert L.nys_proj_qkv(_X, _W, _Q, _K, _V, *dims, None) == _lib.NYS_E_DEVICE
    assert L.nys_proj_out(_X, _W, _Q, *dims, None) == _lib.NYS_E_DEVICE


def test_flash_validation_without_gpu():
    L = _lib.lib()
    ws = 0x50000000
    assert L.nys_flash_workspace_bytes(1, 1, 100, 48, 64, 0) == 0            # d not built
    assert L.nys_flash_workspace_bytes(1, 1, 100, 64, 96, 0) == 0            # chunk not built
    nb = L.nys_flash_workspace_bytes(2, 2, 1000, 64, 128, 1)
    assert nb >= 2 * 2 * 8 * 64 * 64 * 4
    args = (_X, _W, _Q, _K, 2, 2, 1000, 64, 128, 1, ws, nb, None)
    assert L.nys_flash_attention(*args[:10], ws, nb - 1, None) == _lib.NYS_E_ARG  # too small
    assert L.nys_flash_attention(None, *args[1:]) == _lib.NYS_E_ARG
    assert L.nys_flash_attention(*args[:9], 2, ws, nb, None) == _lib.NYS_E_ARG   # causal = 2
    assert L.nys_flash_attention(*args[:8], 96, 1, ws, nb, None) == _lib.NYS_E_UNSUPPORTED
    import torch
    if not torch.cuda.is_available():
        assert L.nys_flash_attention(*args) == _lib.NYS_E_DEVICE


@pytest.mark.parametrize("args,status", [
    ((1, 1, 64, 32, 8, 33, 6, -1), _lib.NYS_E_ARG),          # bad dtype
    ((1, 1, 64, 32, 128, 33, 6, 1), _lib.NYS_E_ARG),         # m > n
    ((1, 1, 64, 32, 8, 32, 6, 1), _lib.NYS_E_ARG),           # even conv width
    ((1, 1, 64, 48, 8, 33, 6, 1), _lib.NYS_E_UNSUPPORTED),   # d not built
    ((1, 1, 1024, 32, 512, 33, 6, 1), _lib.NYS_E_UNSUPPORTED),  # m > 256
])
def test_noalloc_forward_validates_before_any_device_call(args, status):
    null = ctypes.c_void_p(0)
    st = _lib.lib().nys_attn_forward_noalloc(*args, null, null, null, null, null, None)
    assert st == status
    assert _lib.nys_attn_last_error()
