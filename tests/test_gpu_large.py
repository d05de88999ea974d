"""GPU parity on tensors of 2^31 elements (4 GiB in bf16): element offsets
past the int32 range, on the plain and the workspace entry (bf16; the plain
entry's schedule needs more than its default buffer limit here, so it runs
the per-tile kernels) and the FP8 entry on both of its schedules.  Inputs are
seeded and drawn on the device; the oracle checks three whole heads (first,
middle and last) from the very bits the kernels read."""

import numpy as np
import pytest
import torch

import joint_attention_rope_amd as kl
from helpers import assert_bf16_close, assert_fp8_close, bf16_tensor_to_f64, per_tile_kernels

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
B, S, H, D = 2, 4096, 2048, 128           # B S H D = 2^31
HEADS = [(0, 0), (1, 1023), (1, 2047)]


def positions(seed):
    rng = np.random.default_rng(seed)
    return rng.integers(-50, 600, size=(S, 4)).astype(np.int32)


def head64(t, b, h, fp8_scale=None):
    """float64 [1, S, 1, D] of one (b, h) head of a device tensor."""
    x = t[b:b + 1, :, h:h + 1].contiguous().cpu()
    if fp8_scale is None:
        return bf16_tensor_to_f64(x)
    import oracle
    return oracle.e4m3_decode(x.numpy()) * fp8_scale


def test_bf16_2_pow_31_elements_plain_and_workspace():
    import oracle
    g = torch.Generator(device=DEV).manual_seed(2031)
    q, k, v = (torch.randn(B, S, H, D, device=DEV, generator=g, dtype=torch.bfloat16)
               for _ in range(3))
    pos_np = positions(2031)
    pos = torch.from_numpy(pos_np).to(DEV)
    out = torch.empty_like(q)
    assert kl.klein_attn_workspace_size(B, S, H, D) > kl.KLEIN_DEFAULT_BUFFER_LIMIT
    kl.klein_rope4d_attn_fwd(q, k, v, pos, out)
    out_ws = torch.empty_like(q)
    ws = torch.empty(kl.klein_attn_workspace_size(B, S, H, D), dtype=torch.uint8, device=DEV)
    kl.klein_rope4d_attn_fwd_ws(q, k, v, pos, out_ws, ws)
    torch.cuda.synchronize()
    for b, h in HEADS:
        ref = oracle.attention(head64(q, b, h), head64(k, b, h), head64(v, b, h), pos_np)
        print(f"[case] bf16 2^31 elements, head ({b}, {h})", flush=True)
        assert_bf16_close(head64(out, b, h), ref, f"plain ({b}, {h})")
        assert_bf16_close(head64(out_ws, b, h), ref, f"workspace ({b}, {h})")
    del q, k, v, out, out_ws, ws
    torch.cuda.empty_cache()


def test_fp8_2_pow_31_elements():
    import oracle
    g = torch.Generator(device=DEV).manual_seed(2032)
    scales = (1.0 / 32, 1.0 / 32, 1.0 / 32)          # codes of N(0, 32^2): far inside 448
    codes = [(torch.randn(B, S, H, D, device=DEV, generator=g) / s).to(torch.float8_e4m3fn)
             .view(torch.uint8) for s in scales]
    pos_np = positions(2032)
    pos = torch.from_numpy(pos_np).to(DEV)
    outs = []
    for per_tile in (False, True):
        out = torch.empty(B, S, H, D, dtype=torch.bfloat16, device=DEV)
        with per_tile_kernels(per_tile):
            kl.klein_rope4d_attn_fwd_fp8(*codes, pos, out, *scales)
            torch.cuda.synchronize()
        outs.append(out)
    for b, h in HEADS:
        qh, kh, vh = (head64(c, b, h, s) for c, s in zip(codes, scales))
        ref = oracle.attention(qh, kh, vh, pos_np)
        print(f"[case] fp8 2^31 elements, head ({b}, {h})", flush=True)
        assert_fp8_close(head64(outs[0], b, h), ref, f"fp8 buffer ({b}, {h})")
        assert_fp8_close(head64(outs[1], b, h), ref, f"fp8 per-tile ({b}, {h})")
    del codes, outs, out
    with per_tile_kernels():        # frees the library's buffer
        pass
    torch.cuda.empty_cache()
