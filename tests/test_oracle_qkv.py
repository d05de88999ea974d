"""Pins of the QKV-projection oracle (CPU only): scalar brute force; at zero
positions it is torch's linear layer in float64; feeding its output to the
attention without rotation reproduces the fused attention definition; and
planted mistakes fail a pin."""

import numpy as np
import pytest
import torch

from oracle import attention, qkv_rope4d_proj
from oracle import qkv_proj as qkv_mod
from oracle.brute import qkv_proj_scalar


def case(rng, B, S, C, H, D, bias=True):
    x = rng.standard_normal((B, S, C))
    w = rng.standard_normal((3 * H * D, C)) / np.sqrt(C)
    b = rng.standard_normal(3 * H * D) if bias else None
    pos = rng.integers(-40, 700, size=(S, 4)).astype(np.int32)
    return x, w, b, pos


@pytest.mark.parametrize("bias", [True, False])
def test_brute_force(bias):
    rng = np.random.default_rng(11)
    x, w, b, pos = case(rng, 2, 3, 5, 2, 8, bias)
    ref = [np.array(t) for t in qkv_proj_scalar(x.tolist(), w.tolist(),
                                                None if b is None else b.tolist(), pos.tolist(), 2, 8)]
    out = qkv_rope4d_proj(x, w, b, pos, 2, 8)
    for o, r in zip(out, ref):
        assert np.max(np.abs(o - r)) <= 1e-12


def test_zero_positions_is_torch_linear():
    rng = np.random.default_rng(12)
    x, w, b, pos = case(rng, 2, 7, 48, 3, 16)
    pos[:] = 0
    q, k, v = qkv_rope4d_proj(x, w, b, pos, 3, 16)
    y = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w),
                                   torch.from_numpy(b)).numpy().reshape(2, 7, 3, 3, 16)
    for i, t in enumerate((q, k, v)):
        assert np.max(np.abs(t - y[:, :, i])) <= 1e-12


def test_composition_with_attention():
    # attention of the rotated (q', k') at zero positions (no rotation) equals
    # the fused definition on the unrotated projection at the true positions
    rng = np.random.default_rng(13)
    x, w, b, pos = case(rng, 1, 20, 32, 2, 64)
    q, k, v = qkv_rope4d_proj(x, w, b, pos, 2, 64)
    zero = np.zeros_like(pos)
    raw = (x @ w.T + b).reshape(1, 20, 3, 2, 64)
    fused = attention(raw[:, :, 0], raw[:, :, 1], raw[:, :, 2], pos)
    pre = attention(q, k, v, zero)
    assert np.max(np.abs(fused - pre)) <= 1e-12


@pytest.mark.parametrize("mistake", ["w_not_transposed", "q_k_swapped", "v_rotated", "no_bias"])
def test_planted_mistakes_fail_a_pin(monkeypatch, mistake):
    rng = np.random.default_rng(14)
    x, w, b, pos = case(rng, 1, 4, 6, 1, 8)
    ref = [np.array(t) for t in qkv_proj_scalar(x.tolist(), w.tolist(), b.tolist(),
                                                pos.tolist(), 1, 8)]
    good_rope = qkv_mod.rope4d

    def bad_proj(x_, w_, bias_, pos_, H, D, theta=10000.0):
        if mistake == "w_not_transposed":
            ww = np.asarray(w_).reshape(-1)[: w_.size].reshape(w_.shape[1], w_.shape[0]).T
            return qkv_mod.qkv_rope4d_proj.__wrapped__(x_, ww, bias_, pos_, H, D, theta)
        q, k, v = qkv_mod.qkv_rope4d_proj.__wrapped__(x_, w_, None if mistake == "no_bias"
                                                      else bias_, pos_, H, D, theta)
        if mistake == "q_k_swapped":
            return k, q, v
        if mistake == "v_rotated":
            return q, k, good_rope(v, pos_, theta)
        return q, k, v

    import functools
    orig = qkv_mod.qkv_rope4d_proj
    wrapped = functools.wraps(orig)(bad_proj)
    wrapped.__wrapped__ = orig
    monkeypatch.setattr(qkv_mod, "qkv_rope4d_proj", wrapped)
    out = qkv_mod.qkv_rope4d_proj(x, w, b, pos, 1, 8)
    assert max(np.max(np.abs(o - r)) for o, r in zip(out, ref)) > 1e-6
