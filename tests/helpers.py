"""Shared helpers for the GPU tests: upload seeded inputs, run the library,
compare with the oracle at the tolerances of the hot path.

Tolerances (bf16 inputs, bf16 output): max |gpu - oracle| <= 2e-2 and
||gpu - oracle||_2 / ||oracle||_2 <= 5e-3 over the compared elements.
fp8 inputs: relative L2 <= 6e-2 against the exact attention of the dequantised
codes, and every output row within 0.15 relative L2 of its reference row (a
CPU model of the fp8 kernel's roundings puts the largest row at 0.10 on these
inputs, and at 0.08-0.13 on rows that face one dominant key).  A derivation of why these bound the kernel's rounding (bf16 Q'/K'/P and
output, e4m3 Q'/K'/P) is in the design notes.
"""

import contextlib

import numpy as np
import torch

import joint_attention_rope_amd as kl
from workloads import Inputs

# The two schedules of klein_rope4d_attn_fwd / _fp8: "buffer" (the default:
# keys rotated once and the split-KV schedule, in the library's buffer) and
# "per-tile" (buffer limit 0: the kernels that rotate each key tile they load
# and need no memory, as under graph capture or above the limit).
PATHS = ("buffer", "per-tile")

BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
FP8_REL_L2 = 6e-2
FP8_ROW_REL_L2 = 0.15


def to_device(inp: Inputs, dev="cuda:0"):
    """(q, k, v, pos) as GPU tensors holding the generator's exact bits."""
    if inp.descale is None:
        conv = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        conv = lambda a: torch.from_numpy(a).to(dev)
    return conv(inp.q), conv(inp.k), conv(inp.v), torch.from_numpy(inp.pos).to(dev)


def bf16_tensor_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").view(torch.int16).numpy().view(np.uint16).astype(np.uint32) \
        .__lshift__(16).view(np.float32).astype(np.float64)


@contextlib.contextmanager
def per_tile_kernels(on=True):
    """Within the block, klein_rope4d_attn_fwd / _fp8 run the per-tile kernels
    (buffer limit 0); the default limit is restored after it."""
    if not on:
        yield
        return
    kl.klein_set_buffer_limit(0)
    try:
        yield
    finally:
        kl.klein_set_buffer_limit(kl.KLEIN_DEFAULT_BUFFER_LIMIT)


def run_attention(inp: Inputs, dev="cuda:0", path="buffer"):
    """klein_rope4d_attn_fwd (bf16) or klein_rope4d_attn_fwd_fp8 on one of PATHS."""
    assert path in PATHS
    q, k, v, pos = to_device(inp, dev)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    with per_tile_kernels(path == "per-tile"):
        if inp.descale is None:
            kl.klein_rope4d_attn_fwd(q, k, v, pos, out)
        else:
            kl.klein_rope4d_attn_fwd_fp8(q, k, v, pos, out, *inp.descale)
        torch.cuda.synchronize()
    return out


def errors(gpu: np.ndarray, ref: np.ndarray):
    diff = gpu - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    den = float(np.linalg.norm(ref.ravel()))
    rel = float(np.linalg.norm(diff.ravel())) / den if den > 0 else float(np.linalg.norm(diff.ravel()))
    return max_abs, rel


def assert_bf16_close(gpu, ref, what=""):
    max_abs, rel = errors(gpu, ref)
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    assert max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2, \
        f"{what}: max_abs {max_abs:.3e} (<= {BF16_MAX_ABS}), rel_l2 {rel:.3e} (<= {BF16_REL_L2})"
    return max_abs, rel


def sample_rows(S: int, text: int, n: int = 48, seed: int = 0) -> np.ndarray:
    """Query rows to check at full size: both ends, the text/image boundary,
    tile boundaries, and seeded random rows."""
    fixed = {0, 1, S - 1, S - 2, text - 1, text, 255, 256, 257}
    rng = np.random.default_rng(seed)
    fixed |= set(int(x) for x in rng.integers(0, S, size=n))
    return np.array(sorted(r for r in fixed if 0 <= r < S), dtype=np.int64)


def random_inputs(B, S, H, D, seed, pos_lo=-50, pos_hi=600, scale=1.0):
    """Seeded N(0, scale^2) bf16 q, k, v and random integer positions."""
    from workloads import bf16_bits_from_f32, get_config
    rng = np.random.default_rng(seed)
    shape = (B, S, H, D)
    mk = lambda: bf16_bits_from_f32((rng.standard_normal(shape) * scale).astype(np.float32))
    q, k, v = mk(), mk(), mk()
    pos = rng.integers(pos_lo, pos_hi, size=(S, 4)).astype(np.int32)
    return Inputs(get_config(1, B=B, H=H, D=D), q, k, v, pos)


def oracle_full(inp):
    import oracle
    q, k, v = oracle.decode_inputs(inp)
    return oracle.attention(q, k, v, inp.pos)


def oracle_rows(inp, rows):
    import oracle
    return oracle.attention_inputs_rows(inp, rows)


def random_fp8_inputs(B, S, H, D, seed, pos_lo=-50, pos_hi=600, unit_scale=False):
    """Seeded fp8 inputs by the FP8 workload's recipe: N(0,1) rounded to bf16,
    then E4M3 with a per-tensor amax/448 scale (or scale 1 if unit_scale)."""
    from workloads import bf16_bits_from_f32, e4m3_encode, get_config
    rng = np.random.default_rng(seed)
    shape = (B, S, H, D)
    codes, scales = [], []
    for _ in range(3):
        x = rng.standard_normal(shape).astype(np.float32)
        xb = (bf16_bits_from_f32(x).astype(np.uint32) << np.uint32(16)).view(np.float32)
        sc = 1.0 if unit_scale else float(np.float32(np.max(np.abs(xb)) / 448.0))
        codes.append(e4m3_encode(xb.astype(np.float64) / sc))
        scales.append(sc)
    pos = rng.integers(pos_lo, pos_hi, size=(S, 4)).astype(np.int32)
    return Inputs(get_config(5, B=B, H=H, D=D), codes[0], codes[1], codes[2], pos,
                  descale=tuple(scales))


def row_rel_l2(gpu, ref):
    """Relative L2 error of every output row (over the last axis)."""
    den = np.linalg.norm(ref, axis=-1)
    num = np.linalg.norm(gpu - ref, axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def assert_fp8_close(gpu, ref, what=""):
    max_abs, rel = errors(gpu, ref)
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    assert rel <= FP8_REL_L2, f"{what}: rel_l2 {rel:.3e} (<= {FP8_REL_L2}), max_abs {max_abs:.3e}"
    rows = row_rel_l2(gpu, ref)
    worst = np.unravel_index(int(np.argmax(rows)), rows.shape) if rows.size else ()
    assert rows.size == 0 or rows[worst] <= FP8_ROW_REL_L2, \
        f"{what}: row {worst} rel_l2 {rows[worst]:.3e} (<= {FP8_ROW_REL_L2})"
    return max_abs, rel


def assert_elementwise(got, ref, rel, floor, what="", rms_axes=None):
    """|got - ref| <= rel * |ref| + floor * rms(ref) for every element.

    rms(ref) is taken over ``rms_axes`` (kept as broadcast dimensions), e.g.
    over the tokens and channels of each (batch, head) of a [B, S, H, D]
    tensor, or over the whole tensor when None.  The relative term covers the
    final rounding of each element, the floor the error of its sums."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=rms_axes, keepdims=rms_axes is not None))
    excess = np.abs(got - ref) - (rel * np.abs(ref) + floor * rms)
    worst = np.unravel_index(int(np.argmax(excess)), excess.shape) if excess.size else ()
    assert excess.size == 0 or excess[worst] <= 0, (
        f"{what}: element {worst}: got {got[worst]:.6g}, ref {ref[worst]:.6g}, "
        f"bound {rel:g} |ref| + {floor:g} rms")

