"""GPU edge cases beyond the workloads: a sequence longer than 65,535 tokens
with positions outside the kernels' cos/sin tables, odd batch and head
counts, bf16 inputs at the edge of the range the fp16 score operands hold,
and FP8 descales whose product is moderate while each factor is extreme (the
score scale then leaves one E8M0 operand's range and is split) or whose
product is tiny (the softmax must come out uniform)."""

import numpy as np
import pytest
import torch

from helpers import (PATHS, assert_bf16_close, assert_fp8_close, bf16_tensor_to_f64,
                     oracle_full, oracle_rows, random_fp8_inputs, random_inputs, run_attention,
                     sample_rows)
from workloads import Inputs

pytestmark = pytest.mark.gpu


def _rows_of(out, rows):
    return bf16_tensor_to_f64(out[:, torch.from_numpy(rows).to(out.device)])


@pytest.mark.parametrize("path", PATHS)
def test_long_sequence_bf16_sampled_rows(path):
    # S > 65,535 and odd; positions up to 4,000 on every axis, so on the
    # per-tile kernels most keys take the rotation fallback of the bf16
    # kernel's table (positions < 256)
    inp = random_inputs(1, 70001, 2, 64, seed=91, pos_lo=-20, pos_hi=4000)
    out = run_attention(inp, path=path)
    rows = sample_rows(70001, 256, n=32, seed=91)
    assert_bf16_close(_rows_of(out, rows), oracle_rows(inp, rows), "S=70001 bf16")


@pytest.mark.parametrize("path", PATHS)
def test_long_sequence_fp8_sampled_rows(path):
    inp = random_fp8_inputs(1, 70001, 2, 64, seed=92, pos_lo=-20, pos_hi=4000)
    out = run_attention(inp, path=path)
    rows = sample_rows(70001, 256, n=32, seed=92)
    assert_fp8_close(_rows_of(out, rows), oracle_rows(inp, rows), "S=70001 fp8")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("fp8", [False, True])
def test_odd_batch_and_heads_full(fp8, path):
    if fp8:
        inp = random_fp8_inputs(3, 300, 5, 128, seed=93)
        check = assert_fp8_close
    else:
        inp = random_inputs(3, 300, 5, 128, seed=93)
        check = assert_bf16_close
    out = run_attention(inp, path=path)
    check(bf16_tensor_to_f64(out), oracle_full(inp), f"B=3 H=5 fp8={fp8}")


@pytest.mark.parametrize("path", PATHS)
def test_bf16_magnitudes_at_the_stated_range(path):
    # |k| up to 40,000 and |q| up to 300,000 (the stated limits are ~46,000
    # and ~360,000): the rotated, scaled q and k still fit fp16.  The large
    # values sit in channel pairs where the other operand is zero, so the
    # scores stay moderate and the softmax is not one-hot; the result must
    # match the oracle as ordinary inputs do.
    from workloads import bf16_bits_from_f32
    rng = np.random.default_rng(94)
    B, S, H, D = 1, 700, 2, 128
    q = rng.standard_normal((B, S, H, D)).astype(np.float32)
    k = rng.standard_normal((B, S, H, D)).astype(np.float32)
    v = rng.standard_normal((B, S, H, D)).astype(np.float32)
    q[..., 0:2] = 0.0
    k[..., 0:2] = rng.choice([-40000.0, 40000.0], size=(B, S, H, 2))
    k[..., 34:36] = 0.0
    q[..., 34:36] = rng.choice([-300000.0, 300000.0], size=(B, S, H, 2))
    base = random_inputs(B, S, H, D, seed=94)
    inp = Inputs(base.cfg, bf16_bits_from_f32(q), bf16_bits_from_f32(k), bf16_bits_from_f32(v),
                 base.pos)
    out = run_attention(inp, path=path)
    assert_bf16_close(bf16_tensor_to_f64(out), oracle_full(inp), f"large magnitudes {path}")


def _with_descales(inp, dq, dk, dv):
    return Inputs(inp.cfg, inp.q, inp.k, inp.v, inp.pos, descale=(dq, dk, dv))


def test_fp8_score_scale_split_across_operands():
    # dq * dk = 1, but each alone is far outside one E8M0 scale's range
    base = random_fp8_inputs(1, 577, 3, 128, seed=94, unit_scale=True)
    inp = _with_descales(base, 1e-20, 1e20, 0.01)
    ref = oracle_full(inp)
    out = run_attention(inp)
    assert_fp8_close(bf16_tensor_to_f64(out), ref, "dq=1e-20 dk=1e20")
    # the same scores as unit descales: only the product enters the softmax
    out1 = run_attention(_with_descales(base, 1.0, 1.0, 0.01))
    a, b = bf16_tensor_to_f64(out), bf16_tensor_to_f64(out1)
    assert np.max(np.abs(a - b)) <= 2e-3 * max(1e-12, np.max(np.abs(b)))


def test_fp8_tiny_score_scale_gives_mean_of_v():
    # dq = dk = 1e-25: every score underflows to ~0 relative to the others,
    # so each output row is the mean of V (dequantised)
    base = random_fp8_inputs(1, 300, 2, 64, seed=95, unit_scale=True)
    inp = _with_descales(base, 1e-25, 1e-25, 0.5)
    ref = oracle_full(inp)
    mean_v = ref[:, :1].repeat(ref.shape[1], axis=1)
    assert np.max(np.abs(ref - mean_v)) < 1e-9         # the oracle agrees it is uniform
    out = run_attention(inp)
    assert_fp8_close(bf16_tensor_to_f64(out), ref, "dq=dk=1e-25")
