"""Pins of the block-sparse oracle (CPU only): pure-Python brute force on tiny
shapes; every block kept gives the dense oracle; a single kept key block gives
the dense oracle run on that block's keys alone; an empty query block gives
zeros; and plausible mistakes planted in a copy of the oracle fail a pin."""

import numpy as np
import pytest

from oracle import attention, attention_blocksparse
from oracle import blocksparse as bs_mod
from oracle.brute import attention_blocksparse_scalar


def rand_case(rng, B, S, H, D):
    q, k, v = (rng.standard_normal((B, S, H, D)) for _ in range(3))
    pos = rng.integers(-50, 600, size=(S, 4)).astype(np.int32)
    return q, k, v, pos


def rand_mask(rng, B, H, S, qb, kb, p=0.5):
    return (rng.random((B, H, -(-S // qb), -(-S // kb))) < p).astype(np.uint8)


@pytest.mark.parametrize("S,qb,kb", [(7, 4, 2), (13, 4, 3), (16, 8, 4), (5, 5, 5)])
def test_brute_force(S, qb, kb):
    rng = np.random.default_rng(S * 100 + qb * 10 + kb)
    q, k, v, pos = rand_case(rng, 2, S, 2, 8)
    mask = rand_mask(rng, 2, 2, S, qb, kb)
    ref = np.array(attention_blocksparse_scalar(q.tolist(), k.tolist(), v.tolist(),
                                                pos.tolist(), mask.tolist(), qb, kb))
    out = attention_blocksparse(q, k, v, pos, mask, qb, kb)
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_all_blocks_kept_is_dense():
    rng = np.random.default_rng(1)
    q, k, v, pos = rand_case(rng, 1, 300, 2, 64)
    mask = np.ones((1, 2, 2, 5), dtype=np.uint8)
    assert np.max(np.abs(attention_blocksparse(q, k, v, pos, mask, 256, 64)
                         - attention(q, k, v, pos))) <= 1e-13


def test_single_kept_block_is_dense_on_its_keys():
    # one kept key block per query block: the result is the dense definition
    # (the dense oracle's per-head routine) on only that block's keys
    from oracle import joint_attention as dense_mod
    rng = np.random.default_rng(2)
    S, qb, kb = 200, 64, 32
    q, k, v, pos = rand_case(rng, 1, S, 1, 64)
    mask = np.zeros((1, 1, 4, 7), dtype=np.uint8)
    kept = [3, 0, 6, 5]
    for i, j in enumerate(kept):
        mask[0, 0, i, j] = 1
    out = attention_blocksparse(q, k, v, pos, mask, qb, kb)
    for i, j in enumerate(kept):
        qs = np.arange(i * qb, min(S, (i + 1) * qb))
        ks = np.arange(j * kb, min(S, (j + 1) * kb))
        ref = dense_mod._attend_head(q[0, qs, 0], k[0, ks, 0], v[0, ks, 0], pos[qs], pos[ks],
                                     10000.0)
        assert np.max(np.abs(out[0, qs, 0] - ref)) <= 1e-13


def test_empty_query_block_gives_zeros():
    rng = np.random.default_rng(4)
    q, k, v, pos = rand_case(rng, 1, 70, 2, 64)
    mask = rand_mask(rng, 1, 2, 70, 32, 16, p=0.6)
    mask[0, 1, 1, :] = 0
    out = attention_blocksparse(q, k, v, pos, mask, 32, 16)
    assert np.all(out[0, 32:64, 1] == 0)
    assert np.any(out[0, 32:64, 0] != 0)


@pytest.mark.parametrize("mistake", ["transposed_mask", "query_block_off_by_one",
                                     "mask_ignored", "key_block_size_off_by_one"])
def test_planted_mistakes_fail_a_pin(monkeypatch, mistake):
    rng = np.random.default_rng(5)
    S, qb, kb = 13, 4, 3
    q, k, v, pos = rand_case(rng, 1, S, 1, 8)
    mask = rand_mask(rng, 1, 1, S, qb, kb)
    ref = np.array(attention_blocksparse_scalar(q.tolist(), k.tolist(), v.tolist(),
                                                pos.tolist(), mask.tolist(), qb, kb))
    good = bs_mod.key_mask_rows

    def bad(mask_bh, rows, S_, qblock, kblock):
        if mistake == "transposed_mask":
            m = np.zeros((max(mask_bh.shape),) * 2, dtype=mask_bh.dtype)
            m[:mask_bh.shape[1], :mask_bh.shape[0]] = mask_bh.T
            return good(m[:mask_bh.shape[0], :mask_bh.shape[1]], rows, S_, qblock, kblock)
        if mistake == "query_block_off_by_one":
            return good(mask_bh, np.minimum(rows + qblock, S_ - 1), S_, qblock, kblock)
        if mistake == "mask_ignored":
            return np.ones((rows.size, S_), dtype=bool)
        return good(mask_bh, rows, S_, qblock, kblock + 1)

    monkeypatch.setattr(bs_mod, "key_mask_rows", bad)
    out = attention_blocksparse(q, k, v, pos, mask, qb, kb)
    assert np.max(np.abs(out - ref)) > 1e-6
