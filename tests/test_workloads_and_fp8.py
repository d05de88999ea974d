"""Input generator and fp8 codec checks (CPU only).

Token counts are pinned to the pages (tests/golden/token_counts.json); bf16 and
e4m3 rounding are pinned to torch's own casts; the oracle's e4m3 decoder is
pinned on all 256 codes to torch.float8_e4m3fn and to spec values.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import bf16_to_f64, e4m3_decode
from workloads import CONFIGS, bf16_bits_from_f32, e4m3_encode, get_config, make_inputs, make_positions
from workloads.generate import make_float_qkv, outlier_channels

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_token_counts_follow_the_pages():
    g = load("token_counts.json")
    assert g["image_px_1024"] // g["patch_px"] == g["grid_1024"]
    assert g["grid_1024"] ** 2 == g["image_tokens_1024"]
    c2, c3 = CONFIGS[2], CONFIGS[3]
    assert c2.grid == g["grid_1024"]
    assert c2.S - c2.text == g["image_tokens_1024"]
    assert c3.S - c2.S == g["reference_extra_tokens_1024"]
    # 2048 px: twice the side, so a 128 x 128 grid, and so on
    assert CONFIGS[4].grid == 2048 // g["patch_px"]
    assert [CONFIGS[i].S for i in range(1, 6)] == [80, 4608, 8704, 16896, 33280]


def test_flop_counts():
    assert CONFIGS[4].flops == 4 * 2 * 24 * 16896 ** 2 * 128
    assert abs(CONFIGS[4].flops / 1e12 - 7.0158) < 1e-4
    assert abs(CONFIGS[5].flops / 1e12 - 13.6097) < 1e-4


def test_positions_layout():
    pos = make_positions(text=16, grid=8, refs=1)
    assert pos.shape == (16 + 2 * 64, 4) and pos.dtype == np.int32
    assert np.array_equal(pos[:16, 3], np.arange(16))
    assert not pos[:16, :3].any()
    img, ref = pos[16:80], pos[80:]
    assert not img[:, 0].any() and (ref[:, 0] == 1).all()
    assert np.array_equal(img[:, 1:3], ref[:, 1:3])           # shared (h, w)
    assert np.array_equal(img[9], [0, 1, 1, 0])               # h-major raster
    assert not img[:, 3].any()
    # text token 0 and image token (h, w) = (0, 0) both sit at the origin; every
    # other position is distinct
    assert len({tuple(r) for r in pos}) == pos.shape[0] - 1
    assert np.array_equal(pos[0], pos[16])


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * 1e3,
                        np.float32([0, -0.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1e-30, 3e38])])
    ours = bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e4m3_encode_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(300000).astype(np.float32) * 60,
                        np.linspace(-448, 448, 100001, dtype=np.float32),
                        np.float32([0, -0.0, 2 ** -10, 2 ** -10 * 3, 2 ** -6 * 0.96875])])
    ours = e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # saturation (torch's cast does not saturate, the spec's satfinite mode does)
    assert np.array_equal(e4m3_encode(np.array([449.0, 1e9, -7e5])), [0x7E, 0x7E, 0xFE])


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    spec = load("e4m3_spec_values.json")
    for code, val in spec["values"].items():
        got = e4m3_decode(np.array([int(code, 16)], dtype=np.uint8))[0]
        assert got == val and np.signbit(got) == np.signbit(val), code
    for code in spec["nan_codes"]:
        assert np.isnan(e4m3_decode(np.array([int(code, 16)], dtype=np.uint8))[0])
    # encode(decode(c)) round-trips every finite code
    fin = codes[~nan]
    assert np.array_equal(e4m3_encode(e4m3_decode(fin)), fin)


def test_e4m3_code_is_a_log2_of_its_value():
    """The fp8 attention turns scores into probabilities by rounding 8 x + 94 to an
    integer and reading it as an E4M3 code.  That rests on a property of the format:
    a positive normal code c (8..126) encodes 2^(c/8 - 7) times a factor in
    [1, 1 + 0.0616] (linear interpolation inside a binade against the exponential),
    exact at the binade starts; the subnormal codes 1..7 are c * 2^-9, and 0 is zero."""
    codes = np.arange(8, 127)
    vals = e4m3_decode(codes.astype(np.uint8))
    ratio = vals / np.exp2(codes / 8.0 - 7.0)
    assert ratio.min() == 1.0 and ratio.max() < 1.0616
    assert np.all(ratio[codes % 8 == 0] == 1.0)
    # the largest factor, max over f of (1 + f) / 2^f at f = 1/ln 2 - 1, sampled at f = 4/8
    assert abs(ratio.max() - 1.5 / np.sqrt(2.0)) < 1e-12
    # monotone: a larger score never gives a smaller probability
    assert np.all(np.diff(vals) > 0)
    sub = np.arange(0, 8)
    assert np.array_equal(e4m3_decode(sub.astype(np.uint8)), sub * 2.0 ** -9)
    assert e4m3_decode(np.array([126], dtype=np.uint8))[0] == 448.0
    assert np.isnan(e4m3_decode(np.array([127], dtype=np.uint8))[0])


def test_generator_is_seeded_and_follows_recipe():
    a = make_inputs(get_config(1))
    b = make_inputs(get_config(1))
    assert np.array_equal(a.q, b.q) and np.array_equal(a.v, b.v)
    assert a.q.dtype == np.uint16 and a.q.shape == (1, 80, 2, 64)
    q = bf16_to_f64(a.q)
    assert abs(q.mean()) < 0.05 and abs(q.std() - 1) < 0.05


def test_outliers_and_uncond_zeroing():
    cfg = get_config(2, grid=4, text=8)                    # small variant of workload 2
    q, k, v = make_float_qkv(cfg)
    ch = outlier_channels(cfg.H, cfg.D, 2004)
    assert ch.size == 31 and np.unique(ch).size == 31
    kf = k.reshape(cfg.B, cfg.S, -1)
    s = 1 / np.sqrt(cfg.D)
    # outlier channels carry 8x the prescaled std; others the prescaled std
    assert abs(np.std(kf[..., ch]) / s - 8) < 1.0
    mask = np.ones(kf.shape[-1], bool)
    mask[ch] = False
    assert abs(np.std(kf[..., mask]) / s - 1) < 0.1
    cfg4 = get_config(4, grid=4)
    q4, k4, v4 = make_float_qkv(cfg4)
    for arr in (q4, k4, v4):
        assert not arr[1, :cfg4.text].any() and arr[0, :cfg4.text].any()
        assert arr[1, cfg4.text:].any()


def test_fp8_inputs_scales():
    cfg = get_config(5, grid=8, text=16)
    inp = make_inputs(cfg)
    assert inp.q.dtype == np.uint8 and len(inp.descale) == 3
    for codes, sc in zip((inp.q, inp.k, inp.v), inp.descale):
        x = e4m3_decode(codes) * sc
        assert np.isfinite(x).all()
        # amax maps to 448 exactly
        assert abs(np.max(np.abs(e4m3_decode(codes))) - 448.0) == 0.0
