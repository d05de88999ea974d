"""GPU checks of klein_rope4d_attn_fwd_ws, the split-KV schedule.

Query tiles that run whole (the full rounds of the GPU) go through the same
arithmetic as the per-tile kernels (the keys are rotated once before the
call, to the very fp16 values, or e4m3 codes, those kernels form per tile),
so their rows must be bit-identical to them (klein_rope4d_attn_fwd with
buffer limit 0).  Rows of split tiles round P to bf16 relative to each chunk's own
running max and merge fp32 partial sums, so they differ from the dense rows
at the level of the kernel's rounding error; they must match the oracle
within the hot path's tolerances.  Results must not depend on which
workgroup finishes a tile last (repeat calls agree bit for bit), must replay
under graph capture, and the workspace contract (size query, too small a
workspace, none needed) must hold.
"""

import numpy as np
import pytest
import torch

import joint_attention_rope_amd as kl
from helpers import (BF16_MAX_ABS, BF16_REL_L2, assert_bf16_close, assert_fp8_close,
                     bf16_tensor_to_f64, errors, oracle_full, oracle_rows, random_fp8_inputs,
                     random_inputs, run_attention, sample_rows, to_device)
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_ws(inp, dev=DEV):
    q, k, v, pos = to_device(inp, dev)
    B, S, H, D = q.shape
    dtype = kl.KLEIN_DTYPE_BF16 if inp.descale is None else kl.KLEIN_DTYPE_FP8_E4M3
    nbytes = kl.klein_attn_workspace_size(B, S, H, D, dtype)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev) if nbytes else None
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    kl.klein_rope4d_attn_fwd_ws(q, k, v, pos, out, ws, dtype=dtype,
                                descales=inp.descale or (1.0, 1.0, 1.0))
    torch.cuda.synchronize()
    return out, nbytes


def split_rows_mask(B, S, H):
    """[B, S, H] bool: rows of query tiles past the whole rounds (the tiles
    the schedule splits when it needs a workspace)."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    nqt = -(-S // 256)
    items = B * H * nqt
    n_dp = items - items % ncu
    b = np.arange(B)[:, None, None]
    s = np.arange(S)[None, :, None]
    h = np.arange(H)[None, None, :]
    return ((b * H + h) * nqt + s // 256) >= n_dp


@pytest.mark.parametrize("D", [64, 128])
def test_all_tiles_split_matches_oracle(D):
    # 27 query tiles on a GPU of >= 28 compute units: every tile is split
    inp = random_inputs(1, 2100, 3, D, seed=91 + D)
    out, nbytes = run_ws(inp)
    assert nbytes > 0
    assert_bf16_close(bf16_tensor_to_f64(out), oracle_full(inp), f"split-KV D={D}")


def test_fp8_all_tiles_split_matches_oracle():
    inp = random_fp8_inputs(1, 2100, 3, 128, seed=93)
    out, nbytes = run_ws(inp)
    assert nbytes > 0
    assert_fp8_close(bf16_tensor_to_f64(out), oracle_full(inp), "split-KV fp8")


@pytest.mark.parametrize("fp8", [False, True])
def test_whole_rounds_bitwise_and_split_close(fp8):
    B, S, H = 2, 4608, 16                      # 576 query tiles
    inp = (random_fp8_inputs if fp8 else random_inputs)(B, S, H, 128, seed=94)
    out, nbytes = run_ws(inp)
    ref = run_attention(inp, path="per-tile")
    split = split_rows_mask(B, S, H)
    a = out.view(torch.int16).cpu().numpy()
    b = ref.view(torch.int16).cpu().numpy()
    if nbytes == 0:
        assert np.array_equal(a, b)
        return
    assert split.any() and (~split).any()
    assert np.array_equal(a[~split], b[~split]), "whole tiles must equal the dense kernel"
    rows = np.unique(np.nonzero(split.any(axis=(0, 2)))[0])
    rows = rows[np.linspace(0, len(rows) - 1, 24).astype(int)]
    got = bf16_tensor_to_f64(out[:, torch.from_numpy(rows).to(DEV)])
    want = oracle_rows(inp, rows)
    (assert_fp8_close if fp8 else assert_bf16_close)(got, want, "split rows")


def test_workload_4_full_size():
    cfg = get_config(4)
    inp = make_inputs(cfg)
    out, nbytes = run_ws(inp)
    ref = run_attention(inp, path="per-tile")
    assert nbytes > 0
    split = split_rows_mask(cfg.B, cfg.S, cfg.H)
    a = out.view(torch.int16).cpu().numpy()
    b = ref.view(torch.int16).cpu().numpy()
    assert np.array_equal(a[~split], b[~split])
    # split rows: within the hot path's tolerance of the dense kernel, and
    # against the oracle on sampled rows of the split tiles
    max_abs, rel = errors(bf16_tensor_to_f64(out)[split], bf16_tensor_to_f64(ref)[split])
    assert max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2, (max_abs, rel)
    rows = sample_rows(cfg.S, cfg.text, n=24, seed=95)
    rows = np.union1d(rows, np.arange(36 * 256, cfg.S, 997))   # inside the split tiles
    got = bf16_tensor_to_f64(out[:, torch.from_numpy(rows).to(DEV)])
    assert_bf16_close(got, oracle_rows(inp, rows), "workload 4 split-KV")


@pytest.mark.parametrize("D", [64, 128])
def test_value_tiles_ragged_tail(D):
    # 12,345 keys: the bf16 schedule regroups the values into key-major tiles,
    # the last one holding 57 keys and zeros; rows of whole query tiles equal
    # the per-tile kernels (row-major values) bit for bit, split rows and the
    # last rows match the oracle
    B, S, H = 1, 12345, 3
    inp = random_inputs(B, S, H, D, seed=990 + D)
    out, nbytes = run_ws(inp)
    assert nbytes >= B * S * H * D * 2 + B * H * 193 * 64 * D * 2
    ref = run_attention(inp, path="per-tile")
    split = split_rows_mask(B, S, H)
    a = out.view(torch.int16).cpu().numpy()
    b = ref.view(torch.int16).cpu().numpy()
    assert np.array_equal(a[~split], b[~split]), "whole tiles must equal the dense kernel"
    rows = np.unique(np.r_[0, 1, 255, 256, S - 57, S - 2, S - 1, np.arange(5, S, 811)])
    got = bf16_tensor_to_f64(out[:, torch.from_numpy(rows).to(DEV)])
    assert_bf16_close(got, oracle_rows(inp, rows), f"value tiles D={D}")


def test_workload_5_fp8_full_size():
    cfg = get_config(5)
    inp = make_inputs(cfg)
    out, nbytes = run_ws(inp)
    assert nbytes > 0
    rows = sample_rows(cfg.S, cfg.text, n=16, seed=96)
    got = bf16_tensor_to_f64(out[:, torch.from_numpy(rows).to(DEV)])
    assert_fp8_close(got, oracle_rows(inp, rows), "workload 5 split-KV")


def test_repeat_calls_bitwise_identical():
    inp = random_inputs(1, 3000, 5, 128, seed=97)
    a, _ = run_ws(inp)
    b, _ = run_ws(inp)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("D", [64, 128])
def test_unsplit_call_equals_per_tile_kernels(D):
    # S < 2048: nothing is split; the keys are still rotated once into the
    # workspace (fp16, or e4m3 codes for fp8: the values the kernels' cos/sin
    # tables give), so the result equals the dense entry point bit for bit
    # (the values stay row-major below 12,288 keys)
    inp = random_inputs(2, 1000, 3, D, seed=98)
    assert kl.klein_attn_workspace_size(2, 1000, 3, D) == 2 * 1000 * 3 * D * 2
    out, _ = run_ws(inp)
    assert torch.equal(out.view(torch.int16),
                       run_attention(inp, path="per-tile").view(torch.int16))
    inp8 = random_fp8_inputs(1, 1000, 2, D, seed=99)
    assert kl.klein_attn_workspace_size(1, 1000, 2, D, kl.KLEIN_DTYPE_FP8_E4M3) == 1000 * 2 * D
    out8, _ = run_ws(inp8)
    assert torch.equal(out8.view(torch.int16),
                       run_attention(inp8, path="per-tile").view(torch.int16))


def test_workspace_too_small_rejected():
    inp = random_inputs(1, 2100, 3, 128, seed=99)
    q, k, v, pos = to_device(inp)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
    need = kl.klein_attn_workspace_size(1, 2100, 3, 128)
    assert need > 0
    small = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    for ws in (small, None):
        with pytest.raises(kl.KleinError) as e:
            kl.klein_rope4d_attn_fwd_ws(q, k, v, pos, out, ws)
        assert e.value.status == kl.KLEIN_ERR_INVALID_ARG


def test_graph_capture_replays():
    inp = random_inputs(1, 2500, 4, 128, seed=100)
    q, k, v, pos = to_device(inp)
    ref, nbytes = run_ws(inp)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    out = torch.zeros_like(ref)
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            kl.klein_rope4d_attn_fwd_ws(q, k, v, pos, out, ws)
    torch.cuda.synchronize()
    for i in range(4):
        out.zero_()
        ws.fill_(0xAB)                       # stale workspace contents between replays
        run_ws(inp)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i}"


@pytest.mark.parametrize("B,S,H,D,fp8", [(2, 16896, 24, 128, False), (1, 33280, 24, 128, True),
                                         (1, 16896, 4, 128, False), (1, 1000, 3, 64, False),
                                         (1, 12287, 2, 64, False), (1, 12288, 2, 64, False)])
def test_workspace_size_is_keys_plus_planned_partials(B, S, H, D, fp8):
    # the size query on this GPU = the rotated keys (256-aligned), for bf16
    # from 12,288 keys on the key-major value tiles (64 keys each, the last
    # one padded), + the partials of the plan for this GPU's compute-unit count
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    dtype = kl.KLEIN_DTYPE_FP8_E4M3 if fp8 else kl.KLEIN_DTYPE_BF16
    keys = B * S * H * D * (1 if fp8 else 2)
    keys = (keys + 255) // 256 * 256
    values = 0 if fp8 or S < 12288 else B * H * -(-S // 64) * 64 * D * 2
    assert kl.klein_attn_workspace_size(B, S, H, D, dtype) == \
        keys + values + kl.klein_splitkv_plan(B, S, H, D, ncu)[3]
