"""GPU parity: the HIP library against the CPU oracle on the same seeded bits.

Small shapes are compared element by element over the whole output; the
workload shapes are run at full size in the benchmark's launch configuration
and checked on sampled query rows (every batch entry and head), which the
oracle computes one by one.  Each case runs klein_rope4d_attn_fwd on both of
its schedules: the default one in the library's buffer and the per-tile
kernels that need no memory.
"""

import numpy as np
import pytest
import torch

from helpers import (PATHS, assert_bf16_close, bf16_tensor_to_f64, oracle_full, oracle_rows,
                     random_inputs, run_attention, sample_rows)
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu


def _print_case(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("path", PATHS)
def test_tiny_workload_full(path):
    inp = make_inputs(get_config(1))
    _print_case("workload 1", inp.q.shape, path)
    out = bf16_tensor_to_f64(run_attention(inp, path=path))
    assert_bf16_close(out, oracle_full(inp), "workload 1")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S", [1, 2, 17, 63, 64, 65, 255, 256, 257, 300, 577])
def test_ragged_full(S, D, path):
    inp = random_inputs(2, S, 3, D, seed=1000 + S * 7 + D)
    _print_case("ragged", S, D, path)
    out = bf16_tensor_to_f64(run_attention(inp, path=path))
    assert_bf16_close(out, oracle_full(inp), f"S={S} D={D}")


@pytest.mark.parametrize("path", PATHS)
def test_large_positions_full(path):
    """Positions spread over +-4000 on every axis (the documented accuracy range)."""
    inp = random_inputs(1, 200, 2, 128, seed=77, pos_lo=-4000, pos_hi=4000)
    out = bf16_tensor_to_f64(run_attention(inp, path=path))
    assert_bf16_close(out, oracle_full(inp), "large positions")


@pytest.mark.parametrize("cid,overrides", [
    (2, {}),
    (3, {}),
    (4, {}),
    (2, {"text": 480}),     # prompt padded to a multiple of 80 tokens
    (2, {"text": 560}),
    (3, {"refs": 2, "text": 560}),   # two references at t = 1, 2: S = 560 + 3 x 64^2
    (3, {"refs": 3, "text": 480}),   # three references: S = 480 + 4 x 64^2
])
@pytest.mark.parametrize("path", PATHS)
def test_workload_sampled_rows(cid, overrides, path):
    cfg = get_config(cid, **overrides)
    inp = make_inputs(cfg)
    _print_case("workload", cid, overrides, inp.q.shape, path)
    out = run_attention(inp, path=path)
    rows = sample_rows(cfg.S, cfg.text, n=64, seed=cid)
    gpu = bf16_tensor_to_f64(out[:, torch.from_numpy(rows).to(out.device)])
    assert_bf16_close(gpu, oracle_rows(inp, rows), f"workload {cid} {overrides}")


@pytest.mark.parametrize("path", PATHS)
def test_large_magnitudes_within_documented_range(path):
    """Scores run on fp16 operands: |k| up to ~4e4 and |q| up to ~3e5 must work."""
    inp = random_inputs(1, 150, 2, 128, seed=91)
    from workloads import bf16_bits_from_f32
    import oracle
    k = oracle.bf16_to_f64(inp.k) * 3.0e4 / 4.5          # max |k| ~ 3e4
    inp.k = bf16_bits_from_f32(k.astype(np.float32))
    q = oracle.bf16_to_f64(inp.q) * 1.0e-3
    inp.q = bf16_bits_from_f32(q.astype(np.float32))
    out = bf16_tensor_to_f64(run_attention(inp, path=path))
    assert_bf16_close(out, oracle_full(inp), "large |k|")
