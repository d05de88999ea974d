"""Pins of the CPU oracle against things other than itself (CPU only).

* brute force: pure-Python scalar loops on tiny shapes;
* a library special case: all positions zero makes RoPE the identity, so the
  oracle must equal torch's scaled_dot_product_attention in float64;
* closed forms and invariants: each RoPE pair is a 2x2 rotation (orthogonal,
  det 1, norm kept, identity at p = 0, angle p * theta^(-2j/d_a)); scores depend
  only on position differences; softmax rows sum to 1; equal keys give the mean
  of V; S = 1 gives V; token permutation permutes rows; batch/head independence;
* planted mistakes: plausible bugs put into a copy of the oracle must fail at
  least one of the pins above.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import attention, attention_rows, rope4d
from oracle.brute import attention_scalar, rope_scalar
from oracle import joint_attention as attn_mod
from workloads import get_config, make_inputs


def rand_case(rng, B, S, H, D, pos_lo=-50, pos_hi=600):
    q = rng.standard_normal((B, S, H, D))
    k = rng.standard_normal((B, S, H, D))
    v = rng.standard_normal((B, S, H, D))
    pos = rng.integers(pos_lo, pos_hi, size=(S, 4)).astype(np.int32)
    return q, k, v, pos


def brute(q, k, v, pos):
    return np.array(attention_scalar(q.tolist(), k.tolist(), v.tolist(), pos.tolist()))


# ---------------------------------------------------------------- brute force

def test_brute_force_tiny_workload():
    inp = make_inputs(get_config(1))
    q, k, v = oracle.decode_inputs(inp)
    ref = brute(q, k, v, inp.pos)
    out = attention(q, k, v, inp.pos)
    assert np.max(np.abs(out - ref)) <= 1e-12


@pytest.mark.parametrize("S", [1, 2, 3, 17])
@pytest.mark.parametrize("D", [64, 128])
def test_brute_force_random(S, D):
    rng = np.random.default_rng(100 * S + D)
    q, k, v, pos = rand_case(rng, 2, S, 2, D)
    ref = brute(q, k, v, pos)
    assert np.max(np.abs(attention(q, k, v, pos) - ref)) <= 1e-12


def test_rope_brute_force():
    rng = np.random.default_rng(7)
    for D in (8, 64, 128):
        x = rng.standard_normal((5, 3, D))
        pos = rng.integers(-1000, 1000, size=(5, 4))
        y = rope4d(x, pos)
        for s in range(5):
            for h in range(3):
                ref = rope_scalar(x[s, h].tolist(), pos[s].tolist())
                assert np.max(np.abs(y[s, h] - np.array(ref))) <= 1e-12


def test_rows_subset_matches_full():
    rng = np.random.default_rng(3)
    q, k, v, pos = rand_case(rng, 2, 300, 2, 64)
    full = attention(q, k, v, pos)
    rows = np.array([0, 5, 257, 299])
    assert np.max(np.abs(attention_rows(q, k, v, pos, rows) - full[:, rows])) <= 1e-14


# ------------------------------------------------------------ library routine

@pytest.mark.parametrize("S,D", [(1, 64), (80, 64), (300, 128)])
def test_zero_positions_equal_sdpa(S, D):
    rng = np.random.default_rng(S + D)
    q, k, v, _ = rand_case(rng, 2, S, 3, D)
    pos = np.zeros((S, 4), dtype=np.int32)
    out = attention(q, k, v, pos)
    # torch wants [B, H, S, D]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1, 3)))
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))
    ref = ref.numpy().transpose(0, 2, 1, 3)
    assert np.max(np.abs(out - ref)) <= 1e-12


# ------------------------------------------------------- RoPE closed forms

def rope_matrix(D, p):
    """The linear map x -> rope4d(x, p) as a D x D matrix (columns = images of e_i)."""
    eye = np.eye(D)[:, None, :]                     # [D (as S), 1, D]
    pos = np.tile(np.asarray(p)[None, :], (D, 1))
    return rope4d(eye, pos)[:, 0, :].T


@pytest.mark.parametrize("D", [64, 128])
def test_rope_is_rotation(D):
    rng = np.random.default_rng(D)
    for _ in range(5):
        p = rng.integers(-5000, 5000, size=4)
        M = rope_matrix(D, p)
        assert np.max(np.abs(M.T @ M - np.eye(D))) <= 1e-13
        assert abs(np.linalg.det(M) - 1.0) <= 1e-10


def test_rope_identity_and_norm():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((40, 4, 128))
    assert np.array_equal(rope4d(x, np.zeros((40, 4), dtype=np.int32)), x)
    pos = rng.integers(-100000, 100000, size=(40, 4))
    y = rope4d(x, pos)
    # each interleaved pair keeps its own norm
    xp = x.reshape(40, 4, 64, 2)
    yp = y.reshape(40, 4, 64, 2)
    assert np.max(np.abs(np.hypot(*np.moveaxis(xp, -1, 0)) -
                         np.hypot(*np.moveaxis(yp, -1, 0)))) <= 1e-13


@pytest.mark.parametrize("D", [64, 128])
def test_rope_angles_closed_form(D):
    """Basis vector e_{c_a+2j} at p_a = 1 lands on (cos w_j, sin w_j), w_j = 1e4^(-2j/d_a)."""
    da = D // 4
    for a in range(4):
        for j in range(da // 2):
            p = [0, 0, 0, 0]
            p[a] = 3
            x = np.zeros((1, 1, D))
            c = a * da + 2 * j
            x[0, 0, c] = 1.0
            y = rope4d(x, np.array([p]))[0, 0]
            w = 10000.0 ** (-2.0 * j / da)
            expect = np.zeros(D)
            expect[c] = np.cos(3 * w)
            expect[c + 1] = np.sin(3 * w)
            assert np.max(np.abs(y - expect)) <= 1e-15


def test_rope_relative_position():
    rng = np.random.default_rng(5)
    D = 128
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    for _ in range(20):
        p = rng.integers(-600, 600, size=(1, 4))
        pp = rng.integers(-600, 600, size=(1, 4))
        c = rng.integers(-3000, 3000, size=(1, 4))
        a = np.dot(rope4d(q, p)[0, 0], rope4d(k, pp)[0, 0])
        b = np.dot(rope4d(q, p + c)[0, 0], rope4d(k, pp + c)[0, 0])
        assert abs(a - b) <= 1e-10


def test_attention_shift_invariance():
    rng = np.random.default_rng(9)
    q, k, v, pos = rand_case(rng, 1, 200, 2, 128)
    c = np.array([[1, -7, 13, 400]], dtype=np.int32)
    a = attention(q, k, v, pos)
    b = attention(q, k, v, pos + c)
    assert np.max(np.abs(a - b)) <= 1e-10


# --------------------------------------------------------- softmax invariants

def test_v_ones_gives_ones_and_onehot():
    rng = np.random.default_rng(1)
    q, k, _, pos = rand_case(rng, 1, 150, 2, 64)
    v = np.ones_like(q)
    assert np.max(np.abs(attention(q, k, v, pos) - 1.0)) <= 1e-14
    v = np.zeros_like(q)
    v[..., 17] = 1.0
    out = attention(q, k, v, pos)
    assert np.max(np.abs(out[..., 17] - 1.0)) <= 1e-14
    assert np.max(np.abs(np.delete(out, 17, axis=-1))) == 0.0


def test_equal_keys_give_mean_of_v():
    rng = np.random.default_rng(2)
    q, _, v, pos = rand_case(rng, 1, 120, 2, 64)
    k = np.zeros_like(q)                                  # RoPE(0) = 0
    out = attention(q, k, v, pos)
    assert np.max(np.abs(out - v.mean(axis=1, keepdims=True))) <= 1e-14
    # equal keys at one common position (equal after rotation too)
    k = np.tile(rng.standard_normal((1, 1, 2, 64)), (1, 120, 1, 1))
    pos1 = np.tile(rng.integers(0, 50, size=(1, 4)), (120, 1))
    out = attention(q, k, v, pos1)
    assert np.max(np.abs(out - v.mean(axis=1, keepdims=True))) <= 1e-14


def test_single_token_gives_v():
    rng = np.random.default_rng(4)
    q, k, v, pos = rand_case(rng, 2, 1, 3, 128)
    assert np.max(np.abs(attention(q, k, v, pos) - v)) <= 1e-15


def test_permutation_batch_head_independence():
    rng = np.random.default_rng(6)
    q, k, v, pos = rand_case(rng, 2, 90, 3, 64)
    out = attention(q, k, v, pos)
    perm = rng.permutation(90)
    outp = attention(q[:, perm], k[:, perm], v[:, perm], pos[perm])
    assert np.max(np.abs(outp - out[:, perm])) <= 1e-13
    for b in range(2):
        ob = attention(q[b:b + 1], k[b:b + 1], v[b:b + 1], pos)
        assert np.max(np.abs(ob - out[b:b + 1])) <= 1e-15
    oh = attention(q[:, :, 1:2], k[:, :, 1:2], v[:, :, 1:2], pos)
    assert np.max(np.abs(oh - out[:, :, 1:2])) <= 1e-15


# ------------------------------------------------------------ planted mistakes

def _mutant_ropes():
    """Plausible RoPE bugs: each returns a broken rope4d(x, pos, theta)."""
    good = attn_mod.rope4d

    def wrong_sign(x, pos, theta=10000.0):
        return good(x, -np.asarray(pos), theta)

    def half_split(x, pos, theta=10000.0):
        # pairs (j, j + d_a/2) instead of (2j, 2j+1)
        D = x.shape[-1]
        da = D // 4
        idx = np.concatenate([np.stack([a * da + np.arange(da // 2),
                                        a * da + da // 2 + np.arange(da // 2)], -1).ravel()
                              for a in range(4)])
        inv = np.argsort(idx)
        return good(x[..., idx], pos, theta)[..., inv]

    def freq_off_by_one(x, pos, theta=10000.0):
        return good(x, pos, theta ** 1.0625)

    def axes_swapped(x, pos, theta=10000.0):
        return good(x, np.asarray(pos)[:, [1, 0, 2, 3]], theta)

    return [wrong_sign, half_split, freq_off_by_one, axes_swapped]


def _mutant_attends():
    def no_scale(q, k, v, pos_q, pos_k, theta):
        qr = attn_mod.rope4d(q[:, None, :], pos_q, theta)[:, 0, :]
        kr = attn_mod.rope4d(k[:, None, :], pos_k, theta)[:, 0, :]
        s = qr @ kr.T
        e = np.exp(s - s.max(1, keepdims=True))
        return (e / e.sum(1, keepdims=True)) @ v

    def transposed_softmax(q, k, v, pos_q, pos_k, theta):
        qr = attn_mod.rope4d(q[:, None, :], pos_q, theta)[:, 0, :]
        kr = attn_mod.rope4d(k[:, None, :], pos_k, theta)[:, 0, :]
        s = (qr @ kr.T) / np.sqrt(q.shape[-1])
        e = np.exp(s - s.max(0, keepdims=True))
        return (e / e.sum(0, keepdims=True)) @ v

    def rope_on_v(q, k, v, pos_q, pos_k, theta):
        vr = attn_mod.rope4d(v[:, None, :], pos_k, theta)[:, 0, :]
        return _good_attend(q, k, vr, pos_q, pos_k, theta)

    def k_unrotated(q, k, v, pos_q, pos_k, theta):
        qr = attn_mod.rope4d(q[:, None, :], pos_q, theta)[:, 0, :]
        s = (qr @ k.T) / np.sqrt(q.shape[-1])
        e = np.exp(s - s.max(1, keepdims=True))
        return (e / e.sum(1, keepdims=True)) @ v

    return [no_scale, transposed_softmax, rope_on_v, k_unrotated]


_good_attend = attn_mod._attend_head


def _pins_pass():
    """Re-run the core pins against the (possibly patched) oracle."""
    rng = np.random.default_rng(21)
    q, k, v, pos = rand_case(rng, 1, 17, 2, 64)
    if np.max(np.abs(attention(q, k, v, pos) - brute(q, k, v, pos))) > 1e-12:
        return False
    x = rng.standard_normal((3, 1, 64))
    p = rng.integers(-50, 50, size=(3, 4))
    for s in range(3):
        if np.max(np.abs(rope4d(x, p)[s, 0] - np.array(rope_scalar(x[s, 0].tolist(), p[s].tolist())))) > 1e-12:
            return False
    return True


def test_pins_pass_on_good_oracle():
    assert _pins_pass()


@pytest.mark.parametrize("i", range(4))
def test_planted_rope_mistake_is_caught(monkeypatch, i):
    mut = _mutant_ropes()[i]
    monkeypatch.setattr(attn_mod, "rope4d", mut)
    # the attention oracle uses the mutant rope; brute force stays independent
    rng = np.random.default_rng(21)
    q, k, v, pos = rand_case(rng, 1, 17, 2, 64)
    assert np.max(np.abs(attention(q, k, v, pos) - brute(q, k, v, pos))) > 1e-6


@pytest.mark.parametrize("i", range(4))
def test_planted_attention_mistake_is_caught(monkeypatch, i):
    mut = _mutant_attends()[i]
    monkeypatch.setattr(attn_mod, "_attend_head", mut)
    assert not _pins_pass()
