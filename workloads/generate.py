"""Seeded generators for positions, bf16 Q/K/V and fp8-e4m3 codes.

Everything here is input preparation: numbers are drawn, rounded to the storage
format the kernel consumes, and handed out as raw bit patterns.  Seeds follow
seed(workload c, tensor) = 1000*c + {Q: 1, K: 2, V: 3, outlier channels: 4}
with NumPy's PCG64.
"""

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import Config

SEED_Q, SEED_K, SEED_V, SEED_OUTLIERS = 1, 2, 3, 4
E4M3_MAX = 448.0


@dataclass
class Inputs:
    """Host-side inputs of one call.

    q, k, v: uint16 (bf16 bits) or uint8 (e4m3 codes), shape [B, S, H, D]
    pos:     int32 [S, 4], columns (t, h, w, l), shared by every batch entry
    descale: per-tensor (q, k, v) multipliers for fp8 codes, else None
    """
    cfg: Config
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    pos: np.ndarray
    descale: Optional[tuple] = None

    @property
    def dtype(self) -> str:
        return "fp8" if self.descale is not None else "bf16"


def make_positions(text: int, grid: int, refs: int) -> np.ndarray:
    """Positions (t, h, w, l) for [text | image | reference_1 .. reference_R].

    Text token i sits at (0, 0, 0, i).  The output image grid is (0, h, w, 0)
    in h-major raster order; reference r (1-based) repeats the same (h, w)
    grid at t = r, because reference and output share (h, w) coordinates.
    """
    g2 = grid * grid
    S = text + (1 + refs) * g2
    pos = np.zeros((S, 4), dtype=np.int32)
    pos[:text, 3] = np.arange(text, dtype=np.int32)
    hh, ww = np.meshgrid(np.arange(grid, dtype=np.int32),
                         np.arange(grid, dtype=np.int32), indexing="ij")
    for r in range(refs + 1):
        lo = text + r * g2
        pos[lo:lo + g2, 0] = r
        pos[lo:lo + g2, 1] = hh.reshape(-1)
        pos[lo:lo + g2, 2] = ww.reshape(-1)
    return pos


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs here are finite.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    rounded = b + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Encode to OCP FP8 E4M3FN codes: round to nearest even, saturate at 448.

    E4M3FN: sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent
    field 0 holds subnormals m/8 * 2^-6; 0x7F/0xFF are NaN, so the largest
    finite magnitude is 1.75 * 2^8 = 448.  Magnitudes below 2^-6 sit on the
    subnormal grid of step 2^-9 (numpy.rint: ties to even); above it the
    fraction of 2^e * (1 + f) is rounded to 3 bits, ties to the even code.
    Negative inputs keep their sign bit, zero included.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # normal range: drop all but 3 fraction bits of the float64 pattern with
    # round-half-even; a carry out of the fraction bumps the exponent field
    bits = a.view(np.uint64)
    keep = (bits >> np.uint64(49)) & np.uint64(1)
    r = (bits + np.uint64((1 << 48) - 1) + keep) >> np.uint64(49)
    normal = r.astype(np.int64) - ((1023 - 7) << 3)
    # subnormal range: multiples of 2^-9 (code 8 is the smallest normal 2^-6)
    small = a < 2.0 ** -6
    np.copyto(normal, np.rint(a * 512.0).astype(np.int64), where=small)
    code = normal.astype(np.uint8)
    code |= np.signbit(x).astype(np.uint8) << np.uint8(7)
    return code


def _normal(shape, seed: int) -> np.ndarray:
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(
        shape, dtype=np.float32)


def outlier_channels(H: int, D: int, seed: int) -> np.ndarray:
    """round(1% of H*D) distinct (h, d) key channels, as flat indices h*D + d."""
    n = int(round(0.01 * H * D))
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.sort(rng.choice(H * D, size=n, replace=False))


def make_float_qkv(cfg: Config, B: Optional[int] = None, S: Optional[int] = None):
    """Float32 Q, K, V for ``cfg`` before storage rounding."""
    B = cfg.B if B is None else B
    S = cfg.S if S is None else S
    shape = (B, S, cfg.H, cfg.D)
    base = 1000 * cfg.cid
    q = _normal(shape, base + SEED_Q)
    k = _normal(shape, base + SEED_K)
    v = _normal(shape, base + SEED_V)
    if cfg.prescale:
        s = np.float32(1.0 / np.sqrt(cfg.D))
        q *= s
        k *= s
        v *= s
    if cfg.outliers:
        # the same channel set serves every workload that asks for outliers
        ch = outlier_channels(cfg.H, cfg.D, 2000 + SEED_OUTLIERS)
        kf = k.reshape(B, S, cfg.H * cfg.D)
        kf[:, :, ch] *= np.float32(8.0)
    if cfg.uncond_zero_text and B > 1:
        for arr in (q, k, v):
            arr[1, :cfg.text] = 0.0
    return q, k, v


def make_inputs(cfg: Config, B: Optional[int] = None) -> Inputs:
    """Seeded inputs for workload ``cfg`` (bf16 bits, or e4m3 codes + scales)."""
    pos = make_positions(cfg.text, cfg.grid, cfg.refs)
    q, k, v = make_float_qkv(cfg, B=B, S=pos.shape[0])
    if cfg.dtype == "bf16":
        return Inputs(cfg, bf16_bits_from_f32(q), bf16_bits_from_f32(k),
                      bf16_bits_from_f32(v), pos)
    # fp8: values are first stored as bf16, then quantised per tensor with
    # scale = amax / 448 (scale 1 for an all-zero tensor)
    codes, scales = [], []
    for arr in (q, k, v):
        xb = bf16_bits_from_f32(arr).astype(np.uint32) << np.uint32(16)
        xf = xb.view(np.float32)
        amax = float(np.max(np.abs(xf))) if xf.size else 0.0
        scale = amax / E4M3_MAX if amax > 0 else 1.0
        flat = xf.reshape(-1)
        out = np.empty(flat.shape, dtype=np.uint8)
        step = 1 << 22
        for i in range(0, flat.size, step):
            out[i:i + step] = e4m3_encode(flat[i:i + step].astype(np.float64) / scale)
        codes.append(out.reshape(xf.shape))
        scales.append(np.float32(scale))
    return Inputs(cfg, codes[0], codes[1], codes[2], pos,
                  descale=tuple(float(s) for s in scales))


def make_block_mask(B: int, H: int, S: int, text: int, keep_frac: float, seed: int,
                    qblock: int = 256, kblock: int = 64, band: tuple = (4, 8)) -> np.ndarray:
    """Seeded synthetic block mask for the block-sparse entry point, uint8
    [B, H, ceil(S/qblock), ceil(S/kblock)] (1 = compute the block).

    The pages give no rule for which query/key combinations a sparsified
    attention keeps, so this stands in for one with a plausible structure:
    every query block keeps all key blocks holding text tokens, a band of key
    blocks around its own position in the token order (band[0] before,
    band[1] after), and a seeded random share ``keep_frac`` of the rest.
    """
    nq, nk = -(-S // qblock), -(-S // kblock)
    rng = np.random.Generator(np.random.PCG64(seed))
    mask = (rng.random((B, H, nq, nk)) < keep_frac).astype(np.uint8)
    mask[..., : -(-text // kblock)] = 1
    for i in range(nq):
        c = (i * qblock) // kblock
        mask[:, :, i, max(0, c - band[0]):c + band[1]] = 1
    return mask
