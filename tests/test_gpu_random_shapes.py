"""GPU parity on a seeded sweep of shapes: batch, sequence length, heads,
head dim, input format and schedule drawn at random (fixed seed), each
compared with the oracle over the whole output at the hot path's tolerances;
the same for the QKV projection and for the backward.

The fixed-shape tests pick the tile boundaries by hand; this sweep covers the
combinations between them (ragged S against both tile sizes, odd head counts
against the split planner, fp8 and bf16 on both schedules) without choosing
them.
"""

import numpy as np
import pytest

from helpers import (PATHS, assert_bf16_close, assert_fp8_close, bf16_tensor_to_f64,
                     oracle_full, random_fp8_inputs, random_inputs, run_attention)

pytestmark = pytest.mark.gpu


def _cases(n=16, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 4))
        H = int(rng.integers(1, 6))
        while B * H > 8:
            H -= 1
        S = int(rng.integers(1, 900))
        D = int(rng.choice([64, 128]))
        fp8 = bool(rng.integers(0, 2))
        path = PATHS[int(rng.integers(0, len(PATHS)))]
        hi = int(rng.choice([600, 4096]))
        out.append(pytest.param(B, S, H, D, fp8, path, hi, 1000 + i,
                                id=f"B{B}-S{S}-H{H}-D{D}-{'fp8' if fp8 else 'bf16'}-{path}"))
    return out


@pytest.mark.parametrize("B,S,H,D,fp8,path,pos_hi,seed", _cases())
def test_random_shape_matches_oracle(B, S, H, D, fp8, path, pos_hi, seed):
    print(f"[case] B={B} S={S} H={H} D={D} fp8={fp8} path={path} pos<{pos_hi}", flush=True)
    if fp8:
        inp = random_fp8_inputs(B, S, H, D, seed=seed, pos_hi=pos_hi)
    else:
        inp = random_inputs(B, S, H, D, seed=seed, pos_hi=pos_hi)
    got = bf16_tensor_to_f64(run_attention(inp, path=path))
    ref = oracle_full(inp)
    what = f"B={B} S={S} H={H} D={D} {path}"
    if fp8:
        assert_fp8_close(got, ref, what)
    else:
        assert_bf16_close(got, ref, what)


def _qkv_cases(n=10, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fp8 = bool(rng.integers(0, 2))
        B = int(rng.integers(1, 4))
        S = int(rng.integers(1, 700))
        H = int(rng.integers(1, 7))
        D = int(rng.choice([64, 128]))
        C = int(rng.integers(1, 9)) * (128 if fp8 else 64)
        bias = bool(rng.integers(0, 2))
        out.append(pytest.param(B, S, C, H, D, bias, fp8, 2000 + i,
                                id=f"B{B}-S{S}-C{C}-H{H}-D{D}-{'bias' if bias else 'nobias'}-"
                                   f"{'fp8' if fp8 else 'bf16'}"))
    return out


@pytest.mark.parametrize("B,S,C,H,D,bias,fp8,seed", _qkv_cases())
def test_random_projection_shape_matches_oracle(B, S, C, H, D, bias, fp8, seed):
    # the projection with its RoPE epilogue: H D below or above 128, partial
    # token and feature tiles, with and without bias
    import oracle
    import torch
    import joint_attention_rope_amd as kl
    from test_gpu_qkv import check_outputs, fp8_case, proj_case, run_proj
    print(f"[case] qkv B={B} S={S} C={C} H={H} D={D} bias={bias} fp8={fp8}", flush=True)
    if fp8:
        dev_args, descales, host = fp8_case(B, S, C, H, D, bias, seed=seed)
        q = torch.empty(B, S, H, D, dtype=torch.float16, device="cuda:0")
        k = torch.empty_like(q)
        v = torch.empty(B, S, H, D, dtype=torch.bfloat16, device="cuda:0")
        kl.klein_qkv_rope4d_proj(*dev_args, q, k, v, descales=descales)
        torch.cuda.synchronize()
    else:
        dev_args, host = proj_case(B, S, C, H, D, bias, seed=seed)
        q, k, v = run_proj(dev_args, B, S, H, D)
    rq, rk, rv = oracle.qkv_rope4d_proj(*host, H, D)
    check_outputs(q, k, v, rq, rk, rv, f"B={B} S={S} C={C} H={H} D={D}", fp8=fp8)


def _bwd_cases(n=6, seed=20261205):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 4))
        S = int(rng.integers(1, 700))
        D = int(rng.choice([64, 128]))
        out.append(pytest.param(B, S, H, D, 3000 + i, id=f"B{B}-S{S}-H{H}-D{D}"))
    return out


@pytest.mark.parametrize("B,S,H,D,seed", _bwd_cases())
def test_random_backward_shape_matches_oracle(B, S, H, D, seed):
    # the training forward's lse and the backward's dq, dk, dv
    import oracle
    from test_gpu_backward import LSE_ABS, check_grads, run_fwd_bwd
    print(f"[case] backward B={B} S={S} H={H} D={D}", flush=True)
    inp = random_inputs(B, S, H, D, seed=seed)
    (_, lse, dq, dk, dv), (q, k, v, dout) = run_fwd_bwd(inp, dout_seed=seed + 1)
    rq, rk, rv, rlse = oracle.attention_backward(q, k, v, inp.pos, dout)
    assert float(np.max(np.abs(lse.cpu().numpy() - rlse))) <= LSE_ABS
    check_grads((dq, dk, dv), (rq, rk, rv), f"B={B} S={S} H={H} D={D}")
