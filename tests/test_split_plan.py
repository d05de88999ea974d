"""The split-KV planner (host logic, no GPU): klein_splitkv_plan against the
rule its header states, for shapes around the benchmark workloads and one
GPU's shares of them, on several compute-unit counts.  The rule is restated
here from the header (items, key tiles, the last round's remainder, the cost
of c chunks per cut item, the 0.85 gain threshold) and searched by brute
force, so a change to the planner that the header does not describe fails."""

import math

import pytest

import joint_attention_rope_amd as kl

PART_FLOATS = {64: 256 * 64 + 1024, 128: 256 * 128 + 1024}


def documented_plan(B, S, H, D, n_cu):
    items = B * H * math.ceil(S / 256)
    nkt = math.ceil(S / 64)
    rem = items % n_cu
    if nkt < 32 or rem == 0:
        return items, 0, 0, 0
    best_c, best = 1, float(nkt)
    c = 2
    while 8 * c <= nkt and c * rem <= 4 * n_cu:
        cost = math.ceil(c * rem / n_cu) * (nkt / c + 6)
        if cost < best:
            best, best_c = cost, c
        c += 1
    if best_c == 1 or best > 0.85 * nkt:
        return items, 0, 0, 0
    return items - rem, rem, best_c, best_c * rem * PART_FLOATS[D] * 4


SHAPES = [
    (2, 16896, 24, 128), (1, 33280, 24, 128), (1, 4608, 24, 128), (1, 8704, 24, 128),
    (1, 16896, 3, 128), (1, 16896, 4, 128), (1, 16896, 6, 128), (2, 16896, 3, 128),
    (2, 16384, 24, 128), (1, 49664, 24, 128), (1, 66048, 24, 128), (1, 2047, 7, 64),
    (1, 2048, 1, 64), (3, 5000, 5, 64), (1, 100, 2, 128), (4, 12345, 2, 64),
]


@pytest.mark.parametrize("n_cu", [256, 304, 80, 1])
@pytest.mark.parametrize("B,S,H,D", SHAPES)
def test_plan_follows_the_documented_rule(B, S, H, D, n_cu):
    assert kl.klein_splitkv_plan(B, S, H, D, n_cu) == documented_plan(B, S, H, D, n_cu)


@pytest.mark.parametrize("B,S,H,D", SHAPES)
def test_plan_invariants(B, S, H, D):
    n_cu = 256
    whole, cut, chunks, nbytes = kl.klein_splitkv_plan(B, S, H, D, n_cu)
    items = B * H * math.ceil(S / 256)
    nkt = math.ceil(S / 64)
    if cut == 0:
        assert (whole, chunks, nbytes) == (items, 0, 0)
        return
    assert whole + cut == items and whole % n_cu == 0 and 0 < cut < n_cu
    assert 2 <= chunks and 8 * chunks <= nkt and chunks * cut <= 4 * n_cu
    assert nbytes == chunks * cut * PART_FLOATS[D] * 4


def test_benchmark_shape_is_cut_and_whole_rounds_are_not():
    # 2 x 24 x 66 = 3,168 items: 96 past 12 whole rounds on 256 compute units
    whole, cut, chunks, _ = kl.klein_splitkv_plan(2, 16896, 24, 128, 256)
    assert (whole, cut) == (3072, 96) and chunks >= 2
    # 2 x 24 x 64 = 3,072 items fill 12 rounds exactly
    assert kl.klein_splitkv_plan(2, 16384, 24, 128, 256) == (3072, 0, 0, 0)
    # one GPU's 3-head share: 198 items, kept whole (the gain rule)
    assert kl.klein_splitkv_plan(1, 16896, 3, 128, 256)[1] == 0


def test_plan_argument_checks():
    for args in [(0, 100, 1, 128, 256), (1, 0, 1, 128, 256), (1, 100, 0, 128, 256),
                 (1, 100, 1, 128, 0)]:
        with pytest.raises(kl.KleinError) as e:
            kl.klein_splitkv_plan(*args)
        assert e.value.status == kl.KLEIN_ERR_INVALID_ARG
    with pytest.raises(kl.KleinError) as e:
        kl.klein_splitkv_plan(1, 100, 1, 96, 256)
    assert e.value.status == kl.KLEIN_ERR_UNSUPPORTED
