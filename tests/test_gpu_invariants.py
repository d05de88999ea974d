"""GPU invariants that hold at any size (and a race check by determinism)."""

import numpy as np
import pytest
import torch

import joint_attention_rope_amd as kl
import oracle
from helpers import (BF16_MAX_ABS, BF16_REL_L2, assert_bf16_close, bf16_tensor_to_f64, errors,
                     random_inputs, run_attention, to_device)
from workloads import bf16_bits_from_f32, get_config, make_inputs

pytestmark = pytest.mark.gpu


def _out(q, k, v, pos):
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    kl.klein_rope4d_attn_fwd(q, k, v, pos, out)
    return out


def test_deterministic_and_batch_independent():
    inp = random_inputs(2, 700, 4, 128, seed=5)
    q, k, v, pos = to_device(inp)
    a = _out(q, k, v, pos)
    b = _out(q, k, v, pos)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # batch entry 1 alone equals its slice of the B = 2 call, bit for bit
    c = _out(q[1:].contiguous(), k[1:].contiguous(), v[1:].contiguous(), pos)
    torch.cuda.synchronize()
    assert torch.equal(a[1:].view(torch.int16), c.view(torch.int16))


def test_position_shift_invariance():
    inp = random_inputs(1, 500, 2, 128, seed=8)
    q, k, v, pos = to_device(inp)
    a = bf16_tensor_to_f64(_out(q, k, v, pos))
    shift = torch.tensor([[1, -3, 5, 100]], dtype=torch.int32, device=pos.device)
    b = bf16_tensor_to_f64(_out(q, k, v, (pos + shift).contiguous()))
    assert_bf16_close(b, a, "shifted positions")


def test_v_ones_and_zero_keys():
    inp = random_inputs(1, 333, 2, 64, seed=9)
    q, k, v, pos = to_device(inp)
    ones = torch.ones_like(v)
    o = bf16_tensor_to_f64(_out(q, k, ones, pos))
    assert np.max(np.abs(o - 1.0)) <= 2 ** -8
    zk = torch.zeros_like(k)
    o = bf16_tensor_to_f64(_out(q, zk, v, pos))
    mean = oracle.bf16_to_f64(inp.v).mean(axis=1, keepdims=True)
    assert_bf16_close(o, np.broadcast_to(mean, o.shape), "zero keys -> mean of V")


def test_token_permutation():
    inp = random_inputs(1, 400, 2, 128, seed=10)
    q, k, v, pos = to_device(inp)
    a = bf16_tensor_to_f64(_out(q, k, v, pos))
    perm = torch.from_numpy(np.random.default_rng(1).permutation(400)).to(q.device)
    b = bf16_tensor_to_f64(_out(q[:, perm].contiguous(), k[:, perm].contiguous(),
                                v[:, perm].contiguous(), pos[perm].contiguous()))
    assert_bf16_close(b, a[:, perm.cpu().numpy()], "permuted tokens")


def test_uncond_rows_equal_mean_of_v():
    """Workload 4's uncond batch: zero text queries attend uniformly -> mean of V."""
    cfg = get_config(4, grid=16)                        # same recipe, 512 + 256 tokens
    inp = make_inputs(cfg)
    out = bf16_tensor_to_f64(run_attention(inp))
    mean = oracle.bf16_to_f64(inp.v[1]).mean(axis=0)    # [H, D]
    got = out[1, :cfg.text]
    assert_bf16_close(got, np.broadcast_to(mean, got.shape), "uncond text rows")


@pytest.mark.parametrize("D", [64, 128])
def test_rope_apply_matches_oracle(D):
    rng = np.random.default_rng(D)
    S, H = 300, 3
    x = bf16_bits_from_f32(rng.standard_normal((2, S, H, D)).astype(np.float32))
    pos = rng.integers(-4000, 4000, size=(S, 4)).astype(np.int32)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    pt = torch.from_numpy(pos).cuda()
    y = torch.empty_like(xt)
    kl.klein_rope4d_apply(xt, pt, y)
    got = bf16_tensor_to_f64(y)
    ref = oracle.rope4d(oracle.bf16_to_f64(x), pos)
    # one bf16 rounding of the result plus fp32 angle / sin / cos error
    tol = np.abs(ref) * 2.0 ** -8 + 2e-4
    assert (np.abs(got - ref) <= tol).all()
    # norm of each interleaved pair is kept to bf16 precision
    xn = np.hypot(*np.moveaxis(oracle.bf16_to_f64(x).reshape(2, S, H, D // 2, 2), -1, 0))
    yn = np.hypot(*np.moveaxis(got.reshape(2, S, H, D // 2, 2), -1, 0))
    assert np.max(np.abs(xn - yn) / np.maximum(xn, 1e-3)) <= 2.0 ** -7
