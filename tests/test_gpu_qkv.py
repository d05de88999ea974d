"""GPU parity of the QKV projection with its RoPE-4D epilogue (bf16 and FP8
operands) and of the attention on pre-rotated queries and keys, each against
the oracle.

Tolerances of the projection: its outputs are fp32 sums rounded once, to
fp16 (q', k': relative rounding error <= 2^-11) or bf16 (v: <= 2^-8), so the
relative L2 error over a tensor is bounded by those with margin: 1e-3 for
q', k' and 5e-3 for v.  Element by element, |got - ref| <= 2^-10 |ref| (twice
fp16's half-ulp bound) or 2^-8 |ref| (bf16), plus a floor in units of the
tensor's rms.  bf16 operands: 2^-14 for v (the fp32 sums), 2^-12 for q' and
k', whose rotation takes sin and cos from the hardware units.  FP8 operands:
2^-11 for all three, because the fp8 MFMA sums a block's products with less
than fp32's precision -- v, which is not rotated, measured up to 1.75e-4 rms
off on elements far below the rms, against < 6e-5 with bf16 operands.  With FP8 operands every
product of two E4M3 values is exact in fp32, so the same bounds hold against
the projection of the decoded codes.  The attention keeps the bf16 bounds of
the hot path.
"""

import numpy as np
import pytest
import torch

import joint_attention_rope_amd as kl
from helpers import BF16_MAX_ABS, BF16_REL_L2, assert_elementwise, bf16_tensor_to_f64, errors
from workloads import bf16_bits_from_f32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def check_outputs(q, k, v, rq, rk, rv, what, fp8=False):
    fqk, fv = (2.0 ** -11, 2.0 ** -11) if fp8 else (2.0 ** -12, 2.0 ** -14)
    for got, ref, bound, elem, floor, name in (
            (f16_to_f64(q), rq, 1e-3, 2.0 ** -10, fqk, "q'"),
            (f16_to_f64(k), rk, 1e-3, 2.0 ** -10, fqk, "k'"),
            (bf16_tensor_to_f64(v), rv, 5e-3, 2.0 ** -8, fv, "v")):
        _, rel = errors(got, ref)
        assert np.isfinite(got).all() and rel <= bound, f"{what} {name}: rel_l2 {rel:.3e} > {bound}"
        assert_elementwise(got, ref, elem, floor, f"{what} {name}")


def bf16_dev(a):
    bits = bf16_bits_from_f32(np.asarray(a, dtype=np.float32))
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV), \
        (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f16_to_f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def proj_case(B, S, C, H, D, bias, seed):
    rng = np.random.default_rng(seed)
    x_t, x = bf16_dev(rng.standard_normal((B, S, C)))
    w_t, w = bf16_dev(rng.standard_normal((3 * H * D, C)) / np.sqrt(C))
    b_t, b = bf16_dev(rng.standard_normal(3 * H * D) * 0.1) if bias else (None, None)
    pos = rng.integers(-50, 600, size=(S, 4)).astype(np.int32)
    return (x_t, w_t, b_t, torch.from_numpy(pos).to(DEV)), (x, w, b, pos)


def run_proj(dev_args, B, S, H, D):
    q = torch.empty(B, S, H, D, dtype=torch.float16, device=DEV)
    k = torch.empty_like(q)
    v = torch.empty(B, S, H, D, dtype=torch.bfloat16, device=DEV)
    kl.klein_qkv_rope4d_proj(*dev_args, q, k, v)
    torch.cuda.synchronize()
    return q, k, v


@pytest.mark.parametrize("B,S,C,H,D,bias", [
    (2, 300, 128, 2, 64, True),      # partial feature and token tiles
    (1, 513, 256, 4, 128, False),
    (1, 1000, 3072, 2, 128, True),   # the hidden size of the bench shape
    (3, 77, 192, 3, 64, True),
])
def test_projection_matches_oracle(B, S, C, H, D, bias):
    import oracle
    dev_args, host = proj_case(B, S, C, H, D, bias, seed=S + C)
    q, k, v = run_proj(dev_args, B, S, H, D)
    rq, rk, rv = oracle.qkv_rope4d_proj(*host, H, D)
    check_outputs(q, k, v, rq, rk, rv, f"bf16 B={B} S={S} C={C}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S", [1, 65, 577])
def test_prerotated_attention_matches_oracle(S, D):
    import oracle
    rng = np.random.default_rng(S * 3 + D)
    shape = (2, S, 3, D)
    q = torch.from_numpy(rng.standard_normal(shape).astype(np.float16)).to(DEV)
    k = torch.from_numpy(rng.standard_normal(shape).astype(np.float16)).to(DEV)
    v_t, v = bf16_dev(rng.standard_normal(shape))
    out = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    kl.klein_attn_fwd_prerotated(q, k, v_t, out)
    torch.cuda.synchronize()
    ref = oracle.attention(f16_to_f64(q), f16_to_f64(k), v, np.zeros((S, 4), dtype=np.int32))
    max_abs, rel = errors(bf16_tensor_to_f64(out), ref)
    assert max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2, (max_abs, rel)


def test_pipeline_matches_fused_definition():
    # projection -> pre-rotated attention, against the fused attention
    # definition of the unrotated projection at the true positions
    import oracle
    B, S, C, H, D = 1, 700, 256, 2, 128
    dev_args, (x, w, b, pos) = proj_case(B, S, C, H, D, True, seed=71)
    q, k, v = run_proj(dev_args, B, S, H, D)
    out = torch.empty(B, S, H, D, dtype=torch.bfloat16, device=DEV)
    kl.klein_attn_fwd_prerotated(q, k, v, out)
    torch.cuda.synchronize()
    y = (x @ w.T + b).reshape(B, S, 3, H, D)
    ref = oracle.attention(y[:, :, 0], y[:, :, 1], y[:, :, 2], pos)
    max_abs, rel = errors(bf16_tensor_to_f64(out), ref)
    assert max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2, (max_abs, rel)


def fp8_case(B, S, C, H, D, bias, seed):
    """E4M3 codes of N(0, 1) x and N(0, 1/C) W with per-tensor amax/448
    scales, and their float64 values (code x descale) for the oracle."""
    import oracle
    from workloads import e4m3_encode
    rng = np.random.default_rng(seed)
    codes, vals, scales = [], [], []
    for shape, sd in (((B, S, C), 1.0), ((3 * H * D, C), 1.0 / np.sqrt(C))):
        a = (rng.standard_normal(shape) * sd).astype(np.float32).astype(np.float64)
        sc = float(np.float32(np.max(np.abs(a)) / 448.0))
        c = e4m3_encode(a / sc)
        codes.append(torch.from_numpy(c).to(DEV))
        vals.append(oracle.e4m3_decode(c) * sc)
        scales.append(sc)
    b_t, b = bf16_dev(rng.standard_normal(3 * H * D) * 0.1) if bias else (None, None)
    pos = rng.integers(-50, 600, size=(S, 4)).astype(np.int32)
    dev = (codes[0], codes[1], b_t, torch.from_numpy(pos).to(DEV))
    return dev, tuple(scales), (vals[0], vals[1], b, pos)


@pytest.mark.parametrize("B,S,C,H,D,bias", [
    (2, 300, 128, 2, 64, True),      # one K step, partial feature and token tiles
    (1, 513, 256, 4, 128, False),
    (1, 1000, 3072, 2, 128, True),   # the hidden size of the bench shape
    (3, 77, 384, 3, 64, True),
])
def test_fp8_projection_matches_oracle(B, S, C, H, D, bias):
    import oracle
    dev_args, descales, host = fp8_case(B, S, C, H, D, bias, seed=S + C + 1)
    q = torch.empty(B, S, H, D, dtype=torch.float16, device=DEV)
    k = torch.empty_like(q)
    v = torch.empty(B, S, H, D, dtype=torch.bfloat16, device=DEV)
    kl.klein_qkv_rope4d_proj(*dev_args, q, k, v, descales=descales)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qkv_rope4d_proj(*host, H, D)
    check_outputs(q, k, v, rq, rk, rv, f"fp8 B={B} S={S} C={C}", fp8=True)


def test_fp8_projection_rejects_bad_descales_and_width():
    dev_args, _, _ = fp8_case(1, 64, 128, 1, 64, False, seed=5)
    q = torch.empty(1, 64, 1, 64, dtype=torch.float16, device=DEV)
    k = torch.empty_like(q)
    v = torch.empty(1, 64, 1, 64, dtype=torch.bfloat16, device=DEV)
    for d in ((0.0, 1.0), (1.0, float("inf")), (-1.0, 1.0)):
        with pytest.raises(kl.KleinError) as e:
            kl.klein_qkv_rope4d_proj(*dev_args, q, k, v, descales=d)
        assert e.value.status == kl.KLEIN_ERR_INVALID_ARG
    x64 = torch.zeros(1, 64, 64, dtype=torch.uint8, device=DEV)     # C = 64: not a multiple of 128
    w64 = torch.zeros(3 * 64, 64, dtype=torch.uint8, device=DEV)
    with pytest.raises(kl.KleinError) as e:
        kl.klein_qkv_rope4d_proj(x64, w64, None, dev_args[3], q, k, v, descales=(1.0, 1.0))
    assert e.value.status == kl.KLEIN_ERR_UNSUPPORTED


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("B,S,C,H,D", [
    (2, 300, 128, 2, 64),     # H D = 128: the epilogue's LDS-staged stores, a partial token tile
    (1, 513, 256, 4, 128),    # the same with D = 128 and a one-token last tile
    (3, 77, 384, 3, 64),      # H D = 192: the direct per-lane stores
])
def test_projection_repeatable(B, S, C, H, D, fp8):
    # every call writes every output element, and the same bits each time:
    # outputs start from NaN or from whatever memory held, alternately
    if fp8:
        dev_args, descales, _ = fp8_case(B, S, C, H, D, True, seed=900 + S)
        kw = {"descales": descales}
    else:
        dev_args, _ = proj_case(B, S, C, H, D, True, seed=900 + S)
        kw = {}
    first = None
    for i in range(8):
        print(f"[case] repeat {i} B={B} S={S} C={C} H={H} D={D} fp8={fp8}", flush=True)
        make = (lambda *a, **k: torch.full(*a, float("nan"), **k)) if i % 2 else torch.empty
        q = make((B, S, H, D), dtype=torch.float16, device=DEV)
        k = make((B, S, H, D), dtype=torch.float16, device=DEV)
        v = make((B, S, H, D), dtype=torch.bfloat16, device=DEV)
        kl.klein_qkv_rope4d_proj(*dev_args, q, k, v, **kw)
        torch.cuda.synchronize()
        got = [t.view(torch.int16).clone() for t in (q, k, v)]
        assert all(bool(torch.isfinite(t).all()) for t in (q, k, v)), f"call {i}: non-finite output"
        if first is None:
            first = got
        else:
            for name, a, b in zip("qkv", first, got):
                assert torch.equal(a, b), f"call {i}: {name} differs from the first call"
