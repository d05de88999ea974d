"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects invalid arguments before touching any device."""

import ctypes
import os
import re

import pytest

from joint_attention_rope_amd import _capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "klein_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(klein_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted([
        "klein_rope4d_attn_fwd", "klein_rope4d_attn_fwd_fp8", "klein_rope4d_attn_fwd_blocksparse",
        "klein_rope4d_attn_fwd_blocksparse_ws",
        "klein_qkv_rope4d_proj", "klein_qkv_rope4d_proj_fp8", "klein_attn_fwd_prerotated",
        "klein_rope4d_attn_fwd_ws",
        "klein_attn_workspace_size", "klein_splitkv_plan", "klein_rope4d_attn_fwd_lse",
        "klein_rope4d_attn_fwd_lse_ws",
        "klein_rope4d_attn_bwd", "klein_attn_bwd_workspace_size", "klein_rope4d_apply",
        "klein_rope4d_attn_fwd_noalloc", "klein_set_buffer_limit", "klein_status_string",
        "klein_version"])


def test_header_constants_match_the_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define (KLEIN_\w+) (.+)", text))
    assert eval(consts["KLEIN_DEFAULT_BUFFER_LIMIT"].replace("(size_t)", "")) == \
        _capi.KLEIN_DEFAULT_BUFFER_LIMIT == 2 << 30
    assert eval(consts["KLEIN_NOALLOC_SCRATCH_BYTES"].replace("LL", "")) == \
        _capi.KLEIN_NOALLOC_SCRATCH_BYTES


def test_buffer_limit_needs_no_device_while_no_buffer_is_held():
    # no call has created a buffer in this process, so setting the limit
    # makes no HIP call
    lib = _capi.lib()
    assert lib.klein_set_buffer_limit(0) == _capi.KLEIN_OK
    assert lib.klein_set_buffer_limit(_capi.KLEIN_DEFAULT_BUFFER_LIMIT) == _capi.KLEIN_OK


def test_library_exports_every_declared_symbol():
    lib = _capi.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _capi.SIGNATURES, name


def test_status_strings():
    lib = _capi.lib()
    for code in range(5):
        assert lib.klein_status_string(code)
    assert lib.klein_status_string(99) == b"unknown status"
    assert lib.klein_version() >= 100


FAKE = 0x10000          # 16-byte aligned, never dereferenced: checks fail first


@pytest.mark.parametrize("args,status", [
    ((0, FAKE, FAKE, FAKE, FAKE, 1, 8, 1, 128, 0), _capi.KLEIN_ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, 0, FAKE, 1, 8, 1, 128, 0), _capi.KLEIN_ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 0, 8, 1, 128, 0), _capi.KLEIN_ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 0, 1, 128, 0), _capi.KLEIN_ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 0, 128, 0), _capi.KLEIN_ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 1, 96, 0), _capi.KLEIN_ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 1, 256, 0), _capi.KLEIN_ERR_UNSUPPORTED),
    ((FAKE + 2, FAKE, FAKE, FAKE, FAKE, 1, 8, 1, 128, 0), _capi.KLEIN_ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, FAKE + 8, 1, 8, 1, 64, 0), _capi.KLEIN_ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 1, 128, 7), _capi.KLEIN_ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 2 ** 20, 2 ** 30, 2 ** 10, 128, 0), _capi.KLEIN_ERR_UNSUPPORTED),
])
def test_attn_argument_checks(args, status):
    assert _capi.lib().klein_rope4d_attn_fwd(*args, None) == status


@pytest.mark.parametrize("scales", [(0.0, 1.0, 1.0), (1.0, -1.0, 1.0), (1.0, 1.0, float("nan")),
                                    (1.0, float("inf"), 1.0)])
def test_fp8_descale_checks(scales):
    st = _capi.lib().klein_rope4d_attn_fwd_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 1, 128,
                                               *scales, None)
    assert st == _capi.KLEIN_ERR_INVALID_ARG


def test_rope_apply_checks():
    lib = _capi.lib()
    assert lib.klein_rope4d_apply(0, FAKE, FAKE, 1, 8, 1, 128, None) == _capi.KLEIN_ERR_INVALID_ARG
    assert lib.klein_rope4d_apply(FAKE, FAKE, FAKE, 1, 8, 1, 32, None) == _capi.KLEIN_ERR_UNSUPPORTED
    assert lib.klein_rope4d_apply(FAKE, FAKE, FAKE + 4, 1, 8, 1, 64, None) == _capi.KLEIN_ERR_INVALID_ARG


@pytest.mark.parametrize("args,status", [
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 1, 128, 0, 1.0, 1.0, 1.0, 0), _capi.KLEIN_ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 1, 128, 5, 1.0, 1.0, 1.0, FAKE), _capi.KLEIN_ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 1, 128, 1, 0.0, 1.0, 1.0, FAKE), _capi.KLEIN_ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 1, 96, 0, 1.0, 1.0, 1.0, FAKE), _capi.KLEIN_ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64 * 4096 + 1, 1, 64, 0, 1.0, 1.0, 1.0, FAKE),
     _capi.KLEIN_ERR_UNSUPPORTED),
    ((0, FAKE, FAKE, FAKE, FAKE, 1, 8, 1, 128, 0, 1.0, 1.0, 1.0, FAKE), _capi.KLEIN_ERR_INVALID_ARG),
])
def test_blocksparse_argument_checks(args, status):
    """Null mask, bad dtype, bad fp8 descale, unsupported D, too many key
    blocks (> 4096) and null tensors are rejected before any HIP call."""
    assert _capi.lib().klein_rope4d_attn_fwd_blocksparse(*args, None) == status


def test_qkv_proj_and_prerotated_argument_checks():
    lib = _capi.lib()
    U, I = _capi.KLEIN_ERR_UNSUPPORTED, _capi.KLEIN_ERR_INVALID_ARG
    # x, w, bias, pos, q, k, v, B, S, C, H, D
    ok = (FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, 1, 8, 128, 2, 64)
    bad = [((0,) + ok[1:], I), (ok[:4] + (0,) + ok[5:], I), (ok[:9] + (96,) + ok[10:], U),
           (ok[:11] + (32,), U), (ok[:7] + (0,) + ok[8:], I), (ok[:2] + (FAKE + 4,) + ok[3:], I)]
    for args, st in bad:
        assert lib.klein_qkv_rope4d_proj(*args, None) == st, args
    assert lib.klein_attn_fwd_prerotated(0, FAKE, FAKE, FAKE, 1, 8, 1, 64, None) == I
    assert lib.klein_attn_fwd_prerotated(FAKE, FAKE, FAKE, FAKE, 1, 8, 1, 80, None) == U
    assert lib.klein_attn_fwd_prerotated(FAKE, FAKE, FAKE + 8, FAKE, 1, 8, 1, 64, None) == I


@pytest.mark.parametrize("args,status", [
    # q, k, v, pos, out, B, S, H, D, dtype, descales, workspace, bytes
    ((0, FAKE, FAKE, FAKE, FAKE, 1, 4096, 1, 128, 0, 1.0, 1.0, 1.0, FAKE, 1 << 30),
     _capi.KLEIN_ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4096, 1, 128, 3, 1.0, 1.0, 1.0, FAKE, 1 << 30),
     _capi.KLEIN_ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4096, 1, 96, 0, 1.0, 1.0, 1.0, FAKE, 1 << 30),
     _capi.KLEIN_ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4096, 1, 128, 1, 1.0, 0.0, 1.0, FAKE, 1 << 30),
     _capi.KLEIN_ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4096, 1, 128, 0, 1.0, 1.0, 1.0, FAKE + 16, 1 << 30),
     _capi.KLEIN_ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 0, 4096, 1, 128, 0, 1.0, 1.0, 1.0, FAKE, 1 << 30),
     _capi.KLEIN_ERR_INVALID_ARG),
])
def test_workspace_entry_argument_checks(args, status):
    """Null tensors, bad dtype, unsupported D, bad fp8 descale, a workspace
    not 256-byte aligned and sizes < 1 are rejected before any HIP call."""
    assert _capi.lib().klein_rope4d_attn_fwd_ws(*args, None) == status


def test_workspace_size_checks():
    lib = _capi.lib()
    n = ctypes.c_size_t(7)
    assert lib.klein_attn_workspace_size(1, 4096, 1, 128, 0, None) == _capi.KLEIN_ERR_INVALID_ARG
    assert lib.klein_attn_workspace_size(1, 4096, 1, 96, 0, ctypes.byref(n)) == \
        _capi.KLEIN_ERR_UNSUPPORTED
    assert lib.klein_attn_workspace_size(1, 4096, 0, 128, 0, ctypes.byref(n)) == \
        _capi.KLEIN_ERR_INVALID_ARG
    assert lib.klein_attn_workspace_size(1, 4096, 1, 128, 2, ctypes.byref(n)) == \
        _capi.KLEIN_ERR_INVALID_ARG
    assert n.value == 7                   # untouched on error


def test_backward_argument_checks():
    lib = _capi.lib()
    I, U = _capi.KLEIN_ERR_INVALID_ARG, _capi.KLEIN_ERR_UNSUPPORTED
    n = ctypes.c_size_t(0)
    assert lib.klein_attn_bwd_workspace_size(1, 100, 2, 64, ctypes.byref(n)) == _capi.KLEIN_OK
    need = n.value
    assert need >= 4 * 100 * 2 * 64 + 4 * 2 * 100
    assert lib.klein_attn_bwd_workspace_size(1, 100, 2, 96, ctypes.byref(n)) == U
    assert lib.klein_attn_bwd_workspace_size(0, 100, 2, 64, ctypes.byref(n)) == I
    assert lib.klein_attn_bwd_workspace_size(1, 100, 2, 64, None) == I
    # q, k, v, pos, out, dout, lse, dq, dk, dv, B, S, H, D, workspace, bytes
    ok = [FAKE] * 10 + [1, 100, 2, 64, FAKE, need]
    cases = [(5, 0, I), (6, 0, I), (6, FAKE + 2, I), (7, FAKE + 8, I), (14, 0, I),
             (14, FAKE + 16, I), (15, need - 1, I), (13, 80, U), (10, 0, I)]
    for i, val, st in cases:
        args = list(ok)
        args[i] = val
        assert lib.klein_rope4d_attn_bwd(*args, None) == st, (i, val)
    assert lib.klein_rope4d_attn_fwd_lse(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1, 8, 1, 64, None) == I
    assert lib.klein_rope4d_attn_fwd_lse(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 2, 1, 8, 1, 64,
                                         None) == I
    assert lib.klein_rope4d_attn_fwd_lse(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 1, 80, None) == U


def test_every_entry_point_rejects_wide_heads():
    """H D of 2^22 or more (byte offsets within a tile's rows would pass 32
    bits) and S of 2^29 or more are UNSUPPORTED at every entry point, before
    any HIP call; shapes just below the limits pass the check."""
    lib = _capi.lib()
    U = _capi.KLEIN_ERR_UNSUPPORTED
    H, D = 2 ** 15, 128                      # H D = 2^22
    n = ctypes.c_size_t(0)
    plan = (ctypes.c_int * 8)()
    F = FAKE
    calls = {
        "klein_rope4d_attn_fwd": (F, F, F, F, F, 1, 1, H, D, 0, None),
        "klein_rope4d_attn_fwd_fp8": (F, F, F, F, F, 1, 1, H, D, 1.0, 1.0, 1.0, None),
        "klein_rope4d_attn_fwd_ws": (F, F, F, F, F, 1, 1, H, D, 0, 1.0, 1.0, 1.0, F, 1 << 40, None),
        "klein_rope4d_attn_fwd_noalloc": (F, F, F, F, F, 1, 1, H, D, 0, 1.0, 1.0, 1.0, None),
        "klein_rope4d_attn_fwd_lse": (F, F, F, F, F, F, 1, 1, H, D, None),
        "klein_rope4d_attn_fwd_lse_ws": (F, F, F, F, F, F, 1, 1, H, D, F, 1 << 40, None),
        "klein_rope4d_attn_fwd_blocksparse": (F, F, F, F, F, 1, 1, H, D, 0, 1.0, 1.0, 1.0, F, None),
        "klein_rope4d_attn_fwd_blocksparse_ws": (F, F, F, F, F, 1, 1, H, D, 0, 1.0, 1.0, 1.0, F, F,
                                                 1 << 40, None),
        "klein_rope4d_attn_bwd": (F, F, F, F, F, F, F, F, F, F, 1, 1, H, D, F, 1 << 40, None),
        "klein_attn_workspace_size": (1, 1, H, D, 0, ctypes.byref(n)),
        "klein_attn_bwd_workspace_size": (1, 1, H, D, ctypes.byref(n)),
        "klein_splitkv_plan": (1, 1, H, D, 256, plan, ctypes.byref(n)),
        "klein_qkv_rope4d_proj": (F, F, 0, F, F, F, F, 1, 1, 128, H, D, None),
        "klein_qkv_rope4d_proj_fp8": (F, F, 0, F, F, F, F, 1, 1, 128, H, D, 1.0, 1.0, None),
        "klein_attn_fwd_prerotated": (F, F, F, F, 1, 1, H, D, None),
        "klein_rope4d_apply": (F, F, F, 1, 1, H, D, None),
    }
    for name, args in calls.items():
        assert getattr(lib, name)(*args) == U, name
        # S = 2^29 (pos_thwl's index 4 s + axis would pass 32 bits), H = 1:
        # S is the argument before H, or before C and H in the projections
        long_seq = list(args)
        i = long_seq.index(H)
        si = i - 2 if name.startswith("klein_qkv") else i - 1
        assert long_seq[si] == 1, name
        long_seq[si], long_seq[i] = 2 ** 29, 1
        assert getattr(lib, name)(*long_seq) == U, (name, "S = 2^29")
    # one head fewer is within the limit (this size query needs no device)
    assert lib.klein_attn_bwd_workspace_size(1, 1, H - 1, D, ctypes.byref(n)) == _capi.KLEIN_OK
    assert lib.klein_attn_bwd_workspace_size(1, 2 ** 29 - 1, 1, D, ctypes.byref(n)) == _capi.KLEIN_OK
    # the projection's B S (its token count) in 32 bits
    assert lib.klein_qkv_rope4d_proj(F, F, 0, F, F, F, F, 8, 2 ** 28, 128, 1, 64, None) == U
