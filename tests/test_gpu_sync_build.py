"""Race check: the library against its synchronised copy, bit for bit.

libklein_attn_sync.so holds the same attention kernels compiled with a full
wait on every outstanding memory operation and a workgroup barrier at every
stage boundary of their pipeline step (KLEIN_SYNC_CHECK); nothing else
differs.  A stage that read LDS data before another wave had written it, or
overwrote a buffer another wave still read, would give different bits in the
fast build, so every entry point that runs these kernels must return the same
bits from both: the split-KV schedule (keys rotated once; bf16 values in
key-major tiles from 12,288 keys on), the per-tile kernels with the rotation
in the kernel, the block-sparse kernels, the attention on pre-rotated inputs
and the training forward with lse, on ragged shapes, both head sizes and both
formats.  Each call also runs twice on the fast build (repeat runs must agree
too).
"""

import contextlib

import numpy as np
import pytest
import torch

import joint_attention_rope_amd as kl
from joint_attention_rope_amd import _capi
from helpers import random_fp8_inputs, random_inputs, to_device
from workloads import make_block_mask

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@contextlib.contextmanager
def library(path):
    """The Python binding calls the build at `path` inside the block."""
    saved = _capi._lib
    _capi._lib = _capi.load(path)
    try:
        yield
    finally:
        _capi._lib = saved


def bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t.view(torch.int32)


def both_builds(fn):
    """fn() -> tensors, on the library twice and on the synchronised copy."""
    outs = []
    for path in (_capi.LIB_PATH, _capi.LIB_PATH, _capi.SYNC_LIB_PATH):
        with library(path):
            kl.klein_set_buffer_limit(kl.KLEIN_DEFAULT_BUFFER_LIMIT)
            outs.append([t.clone() for t in fn()])
            torch.cuda.synchronize()
    fast, again, synced = outs
    for a, b, c in zip(fast, again, synced):
        assert torch.isfinite(a.float()).all()
        assert torch.equal(bits(a), bits(b)), "repeat run of the library differs"
        assert torch.equal(bits(a), bits(c)), "library and synchronised copy differ"


def dtype_of(inp):
    return kl.KLEIN_DTYPE_BF16 if inp.descale is None else kl.KLEIN_DTYPE_FP8_E4M3


# the bf16 cases of 12,288 keys or more take the key-major value tiles
CASES = [((2, 2500, 5, 128), False), ((1, 1000, 3, 64), False), ((1, 12500, 2, 128), False),
         ((1, 13001, 1, 64), False), ((1, 2100, 3, 64), True), ((2, 1300, 2, 128), True)]


@pytest.mark.parametrize("shape,fp8", CASES)
def test_workspace_schedule(shape, fp8):
    inp = (random_fp8_inputs if fp8 else random_inputs)(*shape, seed=1100 + shape[1])
    q, k, v, pos = to_device(inp, DEV)
    B, S, H, D = shape
    print(f"[case] workspace schedule {shape} fp8={fp8}", flush=True)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)

    def run():
        ws = torch.empty(max(1, kl.klein_attn_workspace_size(B, S, H, D, dtype_of(inp))),
                         dtype=torch.uint8, device=DEV)
        out.fill_(float("nan"))
        kl.klein_rope4d_attn_fwd_ws(q, k, v, pos, out, ws, dtype=dtype_of(inp),
                                    descales=inp.descale or (1.0, 1.0, 1.0))
        return [out]
    both_builds(run)


@pytest.mark.parametrize("shape,fp8", CASES)
def test_per_tile_kernels(shape, fp8):
    inp = (random_fp8_inputs if fp8 else random_inputs)(*shape, seed=1200 + shape[1])
    q, k, v, pos = to_device(inp, DEV)
    print(f"[case] per-tile kernels {shape} fp8={fp8}", flush=True)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)

    def run():
        kl.klein_set_buffer_limit(0)
        out.fill_(float("nan"))
        if inp.descale is None:
            kl.klein_rope4d_attn_fwd(q, k, v, pos, out)
        else:
            kl.klein_rope4d_attn_fwd_fp8(q, k, v, pos, out, *inp.descale)
        torch.cuda.synchronize()
        kl.klein_set_buffer_limit(kl.KLEIN_DEFAULT_BUFFER_LIMIT)
        return [out]
    both_builds(run)


@pytest.mark.parametrize("fp8", [False, True])
def test_block_sparse(fp8):
    B, S, H, D = 1, 2300, 3, 128
    inp = (random_fp8_inputs if fp8 else random_inputs)(B, S, H, D, seed=1300 + fp8)
    q, k, v, pos = to_device(inp, DEV)
    mask = torch.from_numpy(make_block_mask(B, H, S, 512, 0.4, seed=1301)).to(DEV)
    print(f"[case] block-sparse {(B, S, H, D)} fp8={fp8}", flush=True)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)

    def run():
        ws = torch.empty(max(1, kl.klein_attn_workspace_size(B, S, H, D, dtype_of(inp))),
                         dtype=torch.uint8, device=DEV)
        out.fill_(float("nan"))
        kl.klein_rope4d_attn_fwd_blocksparse(q, k, v, pos, out, mask,
                                             descales=inp.descale or (1.0, 1.0, 1.0),
                                             workspace=ws)
        return [out]
    both_builds(run)


def test_prerotated_and_lse():
    B, S, H, D = 2, 1700, 3, 128
    inp = random_inputs(B, S, H, D, seed=1400)
    q, k, v, pos = to_device(inp, DEV)
    g = torch.Generator(device=DEV).manual_seed(1401)
    qr = torch.randn(B, S, H, D, device=DEV, generator=g).to(torch.float16)
    kr = torch.randn(B, S, H, D, device=DEV, generator=g).to(torch.float16)
    print(f"[case] pre-rotated and lse {(B, S, H, D)}", flush=True)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
    out2 = torch.empty_like(out)
    lse = torch.empty(B, H, S, dtype=torch.float32, device=DEV)

    def run():
        out.fill_(float("nan"))
        kl.klein_attn_fwd_prerotated(qr, kr, v, out)
        ws = torch.empty(kl.klein_attn_workspace_size(B, S, H, D), dtype=torch.uint8, device=DEV)
        out2.fill_(float("nan"))
        lse.fill_(float("nan"))
        kl.klein_rope4d_attn_fwd_lse(q, k, v, pos, out2, lse, workspace=ws)
        return [out, out2, lse]
    both_builds(run)
