"""GPU parity of the attention backward (klein_rope4d_attn_bwd) and of the
training forward's log-sum-exp (klein_rope4d_attn_fwd_lse) against the oracle.

Tolerances.  Each gradient is an fp32 sum rounded once to bf16 (relative
error <= 2^-9); inside, P is rounded to bf16 for dv and ds = p (dp - delta) to
fp16 for dq and dk, and the inputs of the backward (the forward's bf16 out and
fp32 lse) carry the forward's own error.  Measured on seeded N(0, 1) inputs
and on the 1024x1024 workload the relative L2 errors are 1.7e-3 (dq, dk) and
2.0-2.4e-3 (dv); the bound is rel-L2 <= 6e-3 per gradient tensor.  Each
element must also satisfy |got - ref| <= 2^-7 |ref| + 0.02 rms, rms taken over
its (batch, head): a CPU model of the kernels' roundings puts the largest
excess over the rounding term at 0.009 rms.  ds carries a per-head power of
two that keeps it inside fp16's range, so these bounds hold for gradients of
any size; cases with dout scaled by 1e-4, 1e-6 (fine-tuning gradients) and
1e5 check that.  The log-sum-exp is a p-weighted mean of score errors: the scores
come from fp16 rotated q and k (relative 2^-11 each), |q'| |k'| / sqrt(D) ~
sqrt(D) for N(0, 1) inputs, so score errors reach ~1e-3; the bound is 4e-3
absolute.
"""

import numpy as np
import pytest
import torch

import joint_attention_rope_amd as kl
from helpers import assert_elementwise, bf16_tensor_to_f64, errors, random_inputs, to_device
from workloads import bf16_bits_from_f32, get_config, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GRAD_REL_L2 = 6e-3
GRAD_ELEM_REL = 2.0 ** -7
GRAD_ELEM_FLOOR = 0.02
LSE_ABS = 4e-3


def bf16_from_f64(x):
    bits = bf16_bits_from_f32(np.asarray(x, dtype=np.float32))
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV), \
        (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def run_fwd_bwd(inp, dout_seed, dout_scale=1.0):
    """GPU forward (out, lse) and backward on inp; returns the device results
    and the float64 values of the inputs and of dout (N(0, dout_scale^2))."""
    import oracle
    q, k, v, pos = to_device(inp)
    B, S, H, D = q.shape
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, H, S, dtype=torch.float32, device=DEV)
    kl.klein_rope4d_attn_fwd_lse(q, k, v, pos, out, lse)
    rng = np.random.default_rng(dout_seed)
    dout, dout64 = bf16_from_f64(rng.standard_normal(q.shape) * dout_scale)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(kl.klein_attn_bwd_workspace_size(B, S, H, D), dtype=torch.uint8, device=DEV)
    kl.klein_rope4d_attn_bwd(q, k, v, pos, out, dout, lse, dq, dk, dv, ws)
    torch.cuda.synchronize()
    q64, k64, v64 = oracle.decode_inputs(inp)
    return (out, lse, dq, dk, dv), (q64, k64, v64, dout64)


def check_grads(gpu, ref, what):
    worst = {}
    for t, r, name in zip(gpu, ref, ("dq", "dk", "dv")):
        got = bf16_tensor_to_f64(t)
        assert np.isfinite(got).all(), f"{what} {name}: non-finite"
        max_abs, rel = errors(got, r)
        worst[name] = (got, r, rel)
        print(f"{what} {name}: max_abs {max_abs:.3e} rel_l2 {rel:.3e}", flush=True)
    for name, (got, r, rel) in worst.items():
        assert rel <= GRAD_REL_L2, f"{what} {name}: rel_l2 {rel:.3e} > {GRAD_REL_L2}"
        assert_elementwise(got, r, GRAD_ELEM_REL, GRAD_ELEM_FLOOR, f"{what} {name}",
                           rms_axes=(1, 3))


@pytest.mark.parametrize("B,S,H,D", [
    (1, 300, 2, 64),      # ragged query and key tiles
    (2, 577, 3, 128),
    (1, 65, 1, 64),       # one partial key block, two query tiles
    (1, 1000, 2, 128),
])
def test_backward_matches_oracle(B, S, H, D):
    import oracle
    inp = random_inputs(B, S, H, D, seed=S + 7 * D)
    (out, lse, dq, dk, dv), (q, k, v, dout) = run_fwd_bwd(inp, dout_seed=S)
    rq, rk, rv, rlse = oracle.attention_backward(q, k, v, inp.pos, dout)
    lse_err = float(np.max(np.abs(lse.cpu().numpy() - rlse)))
    print(f"B={B} S={S} H={H} D={D} lse max_abs {lse_err:.3e}", flush=True)
    check_grads((dq, dk, dv), (rq, rk, rv), f"B={B} S={S} H={H} D={D}")
    assert lse_err <= LSE_ABS


@pytest.mark.parametrize("dout_scale", [1e-4, 1e-6, 1e5])
def test_backward_gradient_size(dout_scale):
    # fine-tuning gradients are small: with ds rounded to fp16 as it is, most
    # of it would fall into fp16's subnormals at 1e-4 and below (and overflow
    # at 1e5); the per-head scale keeps the error where it is at dout ~ 1
    import oracle
    inp = random_inputs(1, 1000, 2, 128, seed=77)
    (out, lse, dq, dk, dv), (q, k, v, dout) = run_fwd_bwd(inp, dout_seed=78, dout_scale=dout_scale)
    rq, rk, rv, _ = oracle.attention_backward(q, k, v, inp.pos, dout)
    check_grads((dq, dk, dv), (rq, rk, rv), f"dout x {dout_scale:g}")


def test_forward_with_lse_equals_forward():
    inp = random_inputs(2, 700, 3, 128, seed=41)
    q, k, v, pos = to_device(inp)
    a = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
    b = torch.empty_like(a)
    lse = torch.empty(2, 3, 700, dtype=torch.float32, device=DEV)
    kl.klein_rope4d_attn_fwd(q, k, v, pos, a)
    kl.klein_rope4d_attn_fwd_lse(q, k, v, pos, b, lse)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_workload_2_sampled_heads():
    # the 1024x1024 text-to-image shape (S = 4608, H = 24, scaled inputs with
    # x8 outlier key channels); the oracle runs two whole heads
    import oracle
    cfg = get_config(2)
    inp = make_inputs(cfg)
    (out, lse, dq, dk, dv), (q, k, v, dout) = run_fwd_bwd(inp, dout_seed=2)
    for h in (0, 17):
        rq, rk, rv, rlse = oracle.attention_backward(q[:, :, h:h + 1], k[:, :, h:h + 1],
                                                     v[:, :, h:h + 1], inp.pos, dout[:, :, h:h + 1])
        assert np.max(np.abs(lse[:, h:h + 1].cpu().numpy() - rlse)) <= LSE_ABS
        check_grads((dq[:, :, h:h + 1], dk[:, :, h:h + 1], dv[:, :, h:h + 1]), (rq, rk, rv),
                    f"workload 2 head {h}")


def test_repeat_bitwise_identical():
    inp = random_inputs(1, 900, 2, 128, seed=43)
    a, _ = run_fwd_bwd(inp, dout_seed=5)
    b, _ = run_fwd_bwd(inp, dout_seed=5)
    for x, y in zip(a[2:], b[2:]):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_graph_capture_replays():
    # the backward runs dq on a second stream, forked from and joined back into
    # the caller's: captured on a side stream, every replay (with eager calls
    # of the backward in between) writes the eager result bit for bit
    inp = random_inputs(1, 2100, 3, 128, seed=47)
    (out, lse, dq0, dk0, dv0), _ = run_fwd_bwd(inp, dout_seed=9)
    q, k, v, pos = to_device(inp)
    B, S, H, D = q.shape
    rng = np.random.default_rng(9)
    dout, _ = bf16_from_f64(rng.standard_normal(q.shape))
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(kl.klein_attn_bwd_workspace_size(B, S, H, D), dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            kl.klein_rope4d_attn_bwd(q, k, v, pos, out, dout, lse, dq, dk, dv, ws)
    torch.cuda.synchronize()
    for i in range(4):
        for t in (dq, dk, dv):
            t.zero_()
        ws.fill_(0xAB)                       # stale workspace contents between replays
        run_fwd_bwd(inp, dout_seed=9)        # eager backward work in between
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in ((dq, dq0), (dk, dk0), (dv, dv0)):
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {i}"


@pytest.mark.parametrize("B,S,H", [(1, 2500, 4), (2, 900, 3), (1, 12300, 1)])
def test_forward_with_lse_on_the_split_schedule(B, S, H):
    # the workspace variant: tiles that run whole give the same bits as the
    # plain training forward, split tiles match the oracle (out and lse); at
    # 12,300 keys the workspace variant reads the values as key-major tiles
    import oracle
    inp = random_inputs(B, S, H, 128, seed=S + H)
    q, k, v, pos = to_device(inp)
    a = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
    b = torch.empty_like(a)
    la = torch.empty(B, H, S, dtype=torch.float32, device=DEV)
    lb = torch.empty_like(la)
    kl.klein_rope4d_attn_fwd_lse(q, k, v, pos, a, la)
    ws = torch.empty(kl.klein_attn_workspace_size(B, S, H, 128), dtype=torch.uint8, device=DEV)
    kl.klein_rope4d_attn_fwd_lse(q, k, v, pos, b, lb, workspace=ws)
    torch.cuda.synchronize()
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    whole, cut, _, _ = kl.klein_splitkv_plan(B, S, H, 128, ncu)
    nqt = -(-S // 256)
    for item in range(whole):                    # items in (b, h, query tile) order
        bb, hh, t = item // (H * nqt), (item // nqt) % H, item % nqt
        r0, r1 = 256 * t, min(S, 256 * t + 256)
        assert torch.equal(a[bb, r0:r1, hh].view(torch.int16), b[bb, r0:r1, hh].view(torch.int16))
        assert torch.equal(la[bb, hh, r0:r1], lb[bb, hh, r0:r1])
    q64, k64, v64 = oracle.decode_inputs(inp)
    ref = oracle.attention(q64, k64, v64, inp.pos)
    got = bf16_tensor_to_f64(b)
    max_abs, rel = errors(got, ref)
    assert max_abs <= 2e-2 and rel <= 5e-3, (max_abs, rel)
    _, _, _, rlse = oracle.attention_backward(q64, k64, v64, inp.pos, np.zeros_like(q64))
    assert np.max(np.abs(lb.cpu().numpy() - rlse)) <= LSE_ABS
