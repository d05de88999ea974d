"""GPU parity of the FP8 E4M3 path against the oracle on the dequantised codes.

The graded reference is exact attention of what the kernel was given (code x
descale); the tolerance is relative L2 <= 6e-2.
"""

import numpy as np
import pytest
import torch

import joint_attention_rope_amd as kl
from helpers import (assert_fp8_close, bf16_tensor_to_f64, errors, oracle_full, oracle_rows,
                     random_fp8_inputs, run_attention, sample_rows, to_device)
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S", [1, 17, 64, 65, 300, 577])
def test_fp8_ragged_full(S, D):
    inp = random_fp8_inputs(2, S, 3, D, seed=5000 + 7 * S + D)
    print("[case] fp8 ragged", S, D, flush=True)
    out = bf16_tensor_to_f64(run_attention(inp))
    assert_fp8_close(out, oracle_full(inp), f"fp8 S={S} D={D}")


def test_fp8_small_edit_workload_full():
    """The FP8 edit recipe (text + image + reference at t = 1) at 8x8 grids."""
    inp = make_inputs(get_config(5, text=16, grid=8))
    out = bf16_tensor_to_f64(run_attention(inp))
    assert_fp8_close(out, oracle_full(inp), "fp8 small edit")


def test_fp8_dtype_code_path_unit_scales():
    """klein_rope4d_attn_fwd with KLEIN_DTYPE_FP8_E4M3 means descales of 1."""
    inp = random_fp8_inputs(1, 200, 2, 128, seed=11, unit_scale=True)
    q, k, v, pos = to_device(inp)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    kl.klein_rope4d_attn_fwd(q, k, v, pos, out, dtype=kl.KLEIN_DTYPE_FP8_E4M3)
    torch.cuda.synchronize()
    assert_fp8_close(bf16_tensor_to_f64(out), oracle_full(inp), "fp8 unit scales")


def test_fp8_edit_workload_sampled_rows():
    cfg = get_config(5)
    inp = make_inputs(cfg)
    print("[case] fp8 workload 5", inp.q.shape, flush=True)
    out = run_attention(inp)
    rows = sample_rows(cfg.S, cfg.text, n=16, seed=5)
    gpu = bf16_tensor_to_f64(out[:, torch.from_numpy(rows).to(out.device)])
    assert_fp8_close(gpu, oracle_rows(inp, rows), "fp8 workload 5")


def test_fp8_multi_reference_sampled_rows():
    # 1024^2 edit with two references (t = 1, 2) and a prompt padded to 560
    cfg = get_config(5, grid=64, refs=2, text=560)
    inp = make_inputs(cfg)
    print("[case] fp8 multi-reference", inp.q.shape, flush=True)
    out = run_attention(inp)
    rows = sample_rows(cfg.S, cfg.text, n=24, seed=55)
    gpu = bf16_tensor_to_f64(out[:, torch.from_numpy(rows).to(out.device)])
    assert_fp8_close(gpu, oracle_rows(inp, rows), "fp8 multi-reference")


def test_fp8_deterministic():
    inp = random_fp8_inputs(1, 700, 4, 128, seed=3)
    a = run_attention(inp)
    b = run_attention(inp)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
