"""GPU parity of the block-sparse entry point against the block-sparse oracle:
every block kept reproduces the dense kernels bit for bit; random masks
match the oracle within the dense tolerances; query blocks with nothing
kept give zeros; a mask keeping only the ragged last key tile exercises the
tail masking through the kept list; the 2048px workload runs with a
structured mask on sampled rows."""

import numpy as np
import pytest
import torch

import joint_attention_rope_amd as kl
from helpers import (assert_bf16_close, assert_fp8_close, bf16_tensor_to_f64, random_fp8_inputs,
                     random_inputs, run_attention, sample_rows, to_device)
from workloads import get_config, make_block_mask, make_inputs

pytestmark = pytest.mark.gpu
QB, KB = kl.KLEIN_SPARSE_QBLOCK, kl.KLEIN_SPARSE_KBLOCK


def run_sparse(inp, mask, dev="cuda:0", workspace=False):
    q, k, v, pos = to_device(inp, dev)
    B, S, H, D = q.shape
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    m = torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).to(dev)
    ws = None
    if workspace:
        dt = kl.KLEIN_DTYPE_BF16 if inp.descale is None else kl.KLEIN_DTYPE_FP8_E4M3
        ws = torch.empty(kl.klein_attn_workspace_size(B, S, H, D, dt), dtype=torch.uint8,
                         device=dev)
    kl.klein_rope4d_attn_fwd_blocksparse(q, k, v, pos, out, m,
                                         descales=inp.descale or (1.0, 1.0, 1.0), workspace=ws)
    torch.cuda.synchronize()
    return out


def oracle_sparse(inp, mask, rows=None):
    import oracle
    S = inp.q.shape[1]
    rows = np.arange(S) if rows is None else rows
    return oracle.attention_blocksparse_inputs_rows(inp, mask, rows, QB, KB)


def rand_mask(rng, B, H, S, p):
    return (rng.random(kl.blocksparse_mask_shape(B, S, H)) < p).astype(np.uint8)


@pytest.mark.parametrize("fp8", [False, True])
def test_all_blocks_kept_equals_dense_bitwise(fp8):
    inp = (random_fp8_inputs if fp8 else random_inputs)(2, 700, 3, 128, seed=61)
    mask = np.ones(kl.blocksparse_mask_shape(2, 700, 3), dtype=np.uint8)
    a = run_sparse(inp, mask)
    b = run_attention(inp)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S", [65, 577, 1000])
def test_random_mask_bf16(S, D):
    rng = np.random.default_rng(S + D)
    inp = random_inputs(1, S, 2, D, seed=S * 7 + D)
    mask = rand_mask(rng, 1, 2, S, 0.5)
    mask[0, 0, 0, :] = 0                          # one empty query block
    out = bf16_tensor_to_f64(run_sparse(inp, mask))
    ref = oracle_sparse(inp, mask)
    assert np.all(out[0, :min(S, QB), 0] == 0)
    assert_bf16_close(out, ref, f"sparse S={S} D={D}")


@pytest.mark.parametrize("D", [64, 128])
def test_random_mask_fp8(D):
    rng = np.random.default_rng(D)
    inp = random_fp8_inputs(1, 900, 2, D, seed=63 + D)
    mask = rand_mask(rng, 1, 2, 900, 0.4)
    out = bf16_tensor_to_f64(run_sparse(inp, mask))
    assert_fp8_close(out, oracle_sparse(inp, mask), f"sparse fp8 D={D}")


def test_only_ragged_last_key_tile_kept():
    S = 300                                       # last key tile holds keys 256..299
    inp = random_inputs(1, S, 2, 128, seed=64)
    mask = np.zeros(kl.blocksparse_mask_shape(1, S, 2), dtype=np.uint8)
    mask[..., -1] = 1
    out = bf16_tensor_to_f64(run_sparse(inp, mask))
    assert_bf16_close(out, oracle_sparse(inp, mask), "last tile only")


def test_single_tile_lists_and_deterministic():
    # one kept tile per query block (the shortest pipelines), twice
    S = 1100
    inp = random_inputs(1, S, 3, 64, seed=65)
    shape = kl.blocksparse_mask_shape(1, S, 3)
    mask = np.zeros(shape, dtype=np.uint8)
    rng = np.random.default_rng(65)
    for h in range(3):
        for i in range(shape[2]):
            mask[0, h, i, rng.integers(0, shape[3])] = 1
    a = run_sparse(inp, mask)
    b = run_sparse(inp, mask)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert_bf16_close(bf16_tensor_to_f64(a), oracle_sparse(inp, mask), "one tile per block")


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("S,D", [(1000, 128), (577, 64), (4000, 128)])
def test_keys_rotated_once_equals_per_tile_bitwise(S, D, fp8):
    # the workspace variant rotates every key once, to the very values the
    # per-tile rotation forms, so the results agree bit for bit
    rng = np.random.default_rng(S + D + fp8)
    inp = (random_fp8_inputs if fp8 else random_inputs)(2, S, 3, D, seed=S + 3 * D + fp8)
    mask = rand_mask(rng, 2, 3, S, 0.45)
    a = run_sparse(inp, mask)
    b = run_sparse(inp, mask, workspace=True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_workspace_variant_checks_the_workspace():
    inp = random_inputs(1, 300, 2, 128, seed=67)
    q, k, v, pos = to_device(inp)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    m = torch.ones(kl.blocksparse_mask_shape(1, 300, 2), dtype=torch.uint8, device=q.device)
    need = (300 * 2 * 128 * 2 + 255) // 256 * 256
    small = torch.empty(need - 256, dtype=torch.uint8, device=q.device)
    with pytest.raises(kl.KleinError) as e:
        kl.klein_rope4d_attn_fwd_blocksparse(q, k, v, pos, out, m, workspace=small)
    assert e.value.status == kl.KLEIN_ERR_INVALID_ARG
    exact = torch.empty(need, dtype=torch.uint8, device=q.device)
    kl.klein_rope4d_attn_fwd_blocksparse(q, k, v, pos, out, m, workspace=exact)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), run_attention(inp).view(torch.int16))


def test_workload_4_structured_mask_sampled_rows():
    cfg = get_config(4)
    inp = make_inputs(cfg)
    mask = make_block_mask(cfg.B, cfg.H, cfg.S, cfg.text, 0.3, seed=66)
    out = run_sparse(inp, mask)
    rows = sample_rows(cfg.S, cfg.text, n=32, seed=66)
    gpu = bf16_tensor_to_f64(out[:, torch.from_numpy(rows).to(out.device)])
    assert_bf16_close(gpu, oracle_sparse(inp, mask, rows), "workload 4 sparse")
