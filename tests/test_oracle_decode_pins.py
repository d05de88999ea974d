"""Pins of the oracle's storage decoders and row helpers (CPU only).

The GPU parity tests at full size grade against oracle.decode_inputs,
oracle.attention_inputs_rows and oracle.attention_blocksparse_inputs_rows,
which decode one (batch, head) slice of the stored inputs at a time and
compute only sampled query rows.  Each is pinned here to something other than
itself:

* bf16_to_f64 against torch's own bfloat16 -> float64 cast on every one of
  the 65,536 bit patterns (NaN patterns: NaN on both sides);
* decode_inputs against torch's float8_e4m3fn cast times each tensor's own
  descale, with three different descales, per tensor and per (b, h) slice;
* the row helpers, on unsorted and repeated rows, against the dense oracles
  (themselves pinned by brute force) run on tensors decoded by torch;
* planted mistakes (the descales of k and v swapped, the descale left out,
  batch and head swapped in the slicing, rows returned sorted) put into a
  copy of the oracle each fail one of these pins.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import blocksparse as bs_mod
from oracle import joint_attention as attn_mod
from workloads import Inputs, bf16_bits_from_f32, e4m3_encode, get_config


def torch_bf16_to_f64(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def torch_e4m3_to_f64(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def bf16_case(B, S, H, D, seed):
    rng = np.random.default_rng(seed)
    mk = lambda: bf16_bits_from_f32(rng.standard_normal((B, S, H, D)).astype(np.float32))
    pos = rng.integers(-40, 500, size=(S, 4)).astype(np.int32)
    return Inputs(get_config(1, B=B, H=H, D=D), mk(), mk(), mk(), pos)


# three descales far apart, so a swap between tensors changes every value
DESCALES = (0.75 / 448, 3.0 / 448, 0.125 / 448)


def fp8_case(B, S, H, D, seed, descales=DESCALES):
    rng = np.random.default_rng(seed)
    codes = [e4m3_encode(rng.standard_normal((B, S, H, D)) * 120.0) for _ in range(3)]
    pos = rng.integers(-40, 500, size=(S, 4)).astype(np.int32)
    return Inputs(get_config(5, B=B, H=H, D=D), *codes, pos, descale=tuple(descales))


def torch_decode(inp):
    """(q, k, v) float64 [B, S, H, D], decoded by torch's casts."""
    if inp.descale is None:
        return tuple(torch_bf16_to_f64(x) for x in (inp.q, inp.k, inp.v))
    return tuple(torch_e4m3_to_f64(x) * float(np.float32(d))
                 for x, d in zip((inp.q, inp.k, inp.v), inp.descale))


# ---------------------------------------------------------------- decoders

def test_bf16_to_f64_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):              # NaN patterns widen to NaN
        ours = oracle.bf16_to_f64(bits)
    ref = torch_bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 127                      # exponent all ones, fraction != 0
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))   # -0.0 kept


def test_decode_inputs_bf16_per_slice():
    inp = bf16_case(2, 37, 3, 64, seed=1)
    ref = torch_decode(inp)
    full = oracle.decode_inputs(inp)
    for got, r in zip(full, ref):
        assert np.array_equal(got, r)
    for b in range(2):
        for h in range(3):
            for got, r in zip(oracle.decode_inputs(inp, b, h), ref):
                assert np.array_equal(got, r[b, :, h, :])


def test_decode_inputs_fp8_three_descales_per_slice():
    inp = fp8_case(2, 41, 3, 64, seed=2)
    ref = torch_decode(inp)
    full = oracle.decode_inputs(inp)
    for got, r in zip(full, ref):
        assert np.array_equal(got, r)
    for b in range(2):
        for h in range(3):
            sl = oracle.decode_inputs(inp, b, h)
            for i, (got, r) in enumerate(zip(sl, ref)):
                assert got.shape == (41, 64)
                assert np.array_equal(got, r[b, :, h, :]), (b, h, i)
    # batch only / head only slices
    for got, r in zip(oracle.decode_inputs(inp, b=1), ref):
        assert np.array_equal(got, r[1])
    for got, r in zip(oracle.decode_inputs(inp, h=2), ref):
        assert np.array_equal(got, r[:, :, 2, :])


# ------------------------------------------------------------- row helpers

ROWS = np.array([300, 0, 257, 5, 299, 5, 128])       # unsorted, one repeated, across tiles


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_attention_inputs_rows_equals_dense(kind):
    inp = bf16_case(2, 301, 3, 64, seed=3) if kind == "bf16" else fp8_case(2, 301, 3, 64, seed=3)
    q, k, v = torch_decode(inp)
    dense = oracle.attention(q, k, v, inp.pos)
    got = oracle.attention_inputs_rows(inp, ROWS)
    assert got.shape == (2, ROWS.size, 3, 64)
    assert np.max(np.abs(got - dense[:, ROWS])) <= 1e-13


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_attention_blocksparse_inputs_rows_equals_dense(kind):
    S = 301
    inp = bf16_case(2, S, 3, 64, seed=4) if kind == "bf16" else fp8_case(2, S, 3, 64, seed=4)
    rng = np.random.default_rng(5)
    mask = (rng.random((2, 3, 2, 5)) < 0.6).astype(np.uint8)
    mask[0, 1, 1] = 0                                # one query block with nothing kept
    q, k, v = torch_decode(inp)
    dense = oracle.attention_blocksparse(q, k, v, inp.pos, mask, 256, 64)
    got = oracle.attention_blocksparse_inputs_rows(inp, mask, ROWS, 256, 64)
    assert got.shape == (2, ROWS.size, 3, 64)
    assert np.max(np.abs(got - dense[:, ROWS])) <= 1e-13
    assert not got[0, np.flatnonzero(ROWS >= 256), 1].any()


# --------------------------------------------------------- planted mistakes

def _swapped_descales(inp, b=None, h=None):
    # k and v trade descales (a q <-> k swap would be harmless: the scores
    # take the product of the two)
    swapped = Inputs(inp.cfg, inp.q, inp.k, inp.v, inp.pos,
                     descale=None if inp.descale is None else
                     (inp.descale[0], inp.descale[2], inp.descale[1]))
    return _good_decode(swapped, b, h)


def _no_descale(inp, b=None, h=None):
    unit = Inputs(inp.cfg, inp.q, inp.k, inp.v, inp.pos,
                  descale=None if inp.descale is None else (1.0, 1.0, 1.0))
    return _good_decode(unit, b, h)


def _batch_head_swapped(inp, b=None, h=None):
    if b is None or h is None:
        return _good_decode(inp, b, h)
    return _good_decode(inp, h, b)


_good_decode = attn_mod.decode_inputs
MUTANTS = [_swapped_descales, _no_descale, _batch_head_swapped]


def _row_pins_pass():
    """The row-helper pins above, as one predicate (square B = H so that the
    swapped slicing stays in bounds)."""
    for inp in (fp8_case(2, 70, 2, 64, seed=6), bf16_case(2, 70, 2, 64, seed=7)):
        q, k, v = torch_decode(inp)
        rows = np.array([69, 3, 40])
        if np.max(np.abs(oracle.attention_inputs_rows(inp, rows)
                         - oracle.attention(q, k, v, inp.pos)[:, rows])) > 1e-13:
            return False
        mask = np.ones((2, 2, 1, 2), dtype=np.uint8)
        mask[1, 0, 0, 1] = 0
        if np.max(np.abs(oracle.attention_blocksparse_inputs_rows(inp, mask, rows, 256, 64)
                         - oracle.attention_blocksparse(q, k, v, inp.pos, mask, 256, 64)[:, rows])) > 1e-13:
            return False
    return True


def test_row_pins_pass_on_good_oracle():
    assert _row_pins_pass()


@pytest.mark.parametrize("i", range(len(MUTANTS)))
def test_planted_decode_mistake_is_caught(monkeypatch, i):
    monkeypatch.setattr(attn_mod, "decode_inputs", MUTANTS[i])
    monkeypatch.setattr(bs_mod, "decode_inputs", MUTANTS[i])
    assert not _row_pins_pass()


def test_planted_sorted_rows_mistake_is_caught(monkeypatch):
    good = attn_mod.attention_inputs_rows
    monkeypatch.setattr(oracle, "attention_inputs_rows",
                        lambda inp, rows, *a, **kw: good(inp, np.sort(rows), *a, **kw))
    inp = bf16_case(1, 70, 2, 64, seed=8)
    q, k, v = torch_decode(inp)
    rows = np.array([69, 3, 40])
    assert np.max(np.abs(oracle.attention_inputs_rows(inp, rows)
                         - oracle.attention(q, k, v, inp.pos)[:, rows])) > 1e-3
