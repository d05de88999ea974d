"""klein_rope4d_attn_fwd_noalloc: the split-KV attention with the library's
static per-GPU scratch instead of a caller workspace, against
klein_rope4d_attn_fwd_ws (same kernels, so the outputs must be equal bit for
bit) on two calls in a row, the second with a smaller input (the scratch
keeps the first call's contents), for bf16 and fp8; and against the oracle
on sampled rows.  A shape that needs more than the scratch is refused before
any device work."""

import ctypes

import numpy as np
import pytest
import torch

import joint_attention_rope_amd as kl
from joint_attention_rope_amd import _capi
from helpers import (assert_bf16_close, assert_fp8_close, bf16_tensor_to_f64, oracle_rows,
                     random_fp8_inputs, random_inputs, to_device)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def via_abi(inp, dtype):
    """One call of klein_rope4d_attn_fwd_noalloc through the C ABI, and the
    same call of klein_rope4d_attn_fwd_ws with a fresh workspace."""
    q, k, v, pos = to_device(inp, DEV)
    B, S, H, D = q.shape
    descale = inp.descale or (1.0, 1.0, 1.0)
    a = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    b = torch.empty_like(a)
    stream = torch.cuda.current_stream().cuda_stream
    st = _capi.lib().klein_rope4d_attn_fwd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), pos.data_ptr(), a.data_ptr(),
        B, S, H, D, dtype, *descale, stream)
    assert st == _capi.KLEIN_OK, kl.klein_status_string(st)
    ws = torch.empty(max(1, kl.klein_attn_workspace_size(B, S, H, D, dtype)), dtype=torch.uint8,
                     device=DEV)
    kl.klein_rope4d_attn_fwd_ws(q, k, v, pos, b, ws, dtype=dtype, descales=descale)
    torch.cuda.synchronize()
    return a, b


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_noalloc_equals_workspace_entry_on_two_calls(kind):
    make = random_inputs if kind == "bf16" else random_fp8_inputs
    dtype = kl.KLEIN_DTYPE_BF16 if kind == "bf16" else kl.KLEIN_DTYPE_FP8_E4M3
    # first a call that splits its last round (workspace: rotated keys and
    # partials), then a smaller one on the same scratch
    for i, (B, S, H, D) in enumerate([(2, 2500, 5, 128), (1, 700, 3, 64)]):
        inp = make(B, S, H, D, seed=900 + i)
        print(f"[case] noalloc {kind} call {i}: B={B} S={S} H={H} D={D}", flush=True)
        a, b = via_abi(inp, dtype)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"call {i}"
        rows = np.unique(np.r_[0, 255, 256, S - 1, np.arange(3, S, 97)])
        got = bf16_tensor_to_f64(a[:, torch.from_numpy(rows).to(DEV)])
        if kind == "bf16":
            assert_bf16_close(got, oracle_rows(inp, rows), f"noalloc {kind} call {i}")
        else:
            assert_fp8_close(got, oracle_rows(inp, rows), f"noalloc {kind} call {i}")


def test_noalloc_refuses_shapes_beyond_its_scratch():
    B, S, H, D = 4, 16896, 24, 128      # 517 MB even with the values row-major
    need = kl.klein_attn_workspace_size(B, S, H, D)
    assert need > kl.KLEIN_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(16, dtype=torch.uint8, device=DEV)   # never read: refused first
    p = x.data_ptr()
    st = _capi.lib().klein_rope4d_attn_fwd_noalloc(p, p, p, p, p, B, S, H, D,
                                                   kl.KLEIN_DTYPE_BF16, 1.0, 1.0, 1.0, None)
    assert st == _capi.KLEIN_ERR_UNSUPPORTED
    assert "scratch" in kl.klein_status_string(st)
    # the largest fp8 headline shape fits the workspace layout as it is
    assert kl.klein_attn_workspace_size(1, 33280, 24, 128, kl.KLEIN_DTYPE_FP8_E4M3) \
        <= kl.KLEIN_NOALLOC_SCRATCH_BYTES


def test_noalloc_runs_the_bf16_headline_shape():
    # 2048^2 text-to-image with CFG: the workspace entry's layout (rotated keys,
    # values regrouped into key-major tiles, partials) needs more than the
    # scratch, so the call keeps the values row-major and fits; the kernels
    # differ only in how they read V^T, so the outputs are equal bit for bit
    B, S, H, D = 2, 16896, 24, 128
    assert kl.klein_attn_workspace_size(B, S, H, D) > kl.KLEIN_NOALLOC_SCRATCH_BYTES
    print(f"[case] noalloc bf16 B={B} S={S} H={H} D={D}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(905)
    q, k, v = (torch.randn(B, S, H, D, device=DEV, generator=g, dtype=torch.bfloat16)
               for _ in range(3))
    rng = np.random.default_rng(905)
    pos = torch.from_numpy(rng.integers(-50, 600, size=(S, 4)).astype(np.int32)).to(DEV)
    a = torch.full_like(q, float("nan"))
    stream = torch.cuda.current_stream().cuda_stream
    st = _capi.lib().klein_rope4d_attn_fwd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), pos.data_ptr(), a.data_ptr(),
        B, S, H, D, kl.KLEIN_DTYPE_BF16, 1.0, 1.0, 1.0, stream)
    assert st == _capi.KLEIN_OK, kl.klein_status_string(st)
    ws = torch.empty(kl.klein_attn_workspace_size(B, S, H, D), dtype=torch.uint8, device=DEV)
    b = torch.empty_like(q)
    kl.klein_rope4d_attn_fwd_ws(q, k, v, pos, b, ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    del q, k, v, a, b, ws
    torch.cuda.empty_cache()
