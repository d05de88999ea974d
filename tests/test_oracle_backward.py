"""Pins of the backward oracle (oracle/backward.py), all on the CPU:

* central finite differences of the forward oracle -- an independent code
  path -- for dq, dk and dv on small random shapes with random positions;
* the library special case: at zero positions RoPE is the identity, so the
  gradients equal torch.autograd through scaled_dot_product_attention (float64);
* invariants: sum_j dv_j = sum_i dout_i; sum_j R_j dk_j = 0; dq = dk = 0 when
  v is the same for every key; lse = log S when every score is 0; lse against
  scalar loops;
* planted mistakes (back-rotation by +p instead of -p, a dropped delta term,
  a dropped softmax scale, dk from ds instead of its transpose) must each fail
  a pin.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.backward as bwd_mod
from oracle import attention, rope4d
from oracle.backward import attention_backward


def case(seed, B, S, H, D, pos_lo=-40, pos_hi=300):
    rng = np.random.default_rng(seed)
    q, k, v, dout = (rng.standard_normal((B, S, H, D)) for _ in range(4))
    pos = rng.integers(pos_lo, pos_hi, size=(S, 4)).astype(np.int32)
    return q, k, v, dout, pos


def finite_differences(q, k, v, dout, pos, h=1e-5):
    """Central differences of L = sum(dout * attention(q, k, v)) for every
    element of q, k and v."""
    loss = lambda a, b, c: float(np.sum(dout * attention(a, b, c, pos, workers=1)))
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        g = np.empty_like(args[which])
        for idx in np.ndindex(*g.shape):
            x = args[which]
            x0 = x[idx]
            x[idx] = x0 + h
            lp = loss(*args)
            x[idx] = x0 - h
            lm = loss(*args)
            x[idx] = x0
            g[idx] = (lp - lm) / (2 * h)
        grads.append(g)
    return grads


@pytest.mark.parametrize("seed,S,D", [(1, 5, 8), (2, 4, 16)])
def test_finite_differences(seed, S, D):
    q, k, v, dout, pos = case(seed, 1, S, 2, D)
    dq, dk, dv, _ = attention_backward(q, k, v, pos, dout, workers=1)
    fq, fk, fv = finite_differences(q, k, v, dout, pos)
    for got, want, name in ((dq, fq, "dq"), (dk, fk, "dk"), (dv, fv, "dv")):
        assert np.max(np.abs(got - want)) <= 1e-7 * max(1.0, np.max(np.abs(want))), name


def test_zero_positions_match_torch_autograd():
    q, k, v, dout, _ = case(3, 2, 37, 3, 64)
    pos = np.zeros((37, 4), dtype=np.int32)
    dq, dk, dv, _ = attention_backward(q, k, v, pos, dout)
    tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3), dtype=torch.float64, requires_grad=True)
                  for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    out.backward(torch.tensor(dout.transpose(0, 2, 1, 3), dtype=torch.float64))
    for got, t in ((dq, tq), (dk, tk), (dv, tv)):
        want = t.grad.numpy().transpose(0, 2, 1, 3)
        assert np.max(np.abs(got - want)) <= 1e-12


def test_invariants():
    q, k, v, dout, pos = case(4, 2, 50, 2, 64)
    dq, dk, dv, lse = attention_backward(q, k, v, pos, dout)
    # rows of p sum to 1
    assert np.max(np.abs(dv.sum(axis=1) - dout.sum(axis=1))) <= 1e-11
    # softmax is unchanged by a shift of a row's scores: sum_j dk'_j = 0
    assert np.max(np.abs(rope4d(dk, pos).sum(axis=1))) <= 1e-11
    # v the same for every key: the output does not depend on q or k
    vc = np.broadcast_to(v[:, :1], v.shape).copy()
    dq0, dk0, _, _ = attention_backward(q, k, vc, pos, dout)
    assert np.max(np.abs(dq0)) <= 1e-12 and np.max(np.abs(dk0)) <= 1e-12
    # every score 0: lse = log S
    _, _, _, lse0 = attention_backward(np.zeros_like(q), k, v, pos, dout)
    assert np.max(np.abs(lse0 - math.log(50))) <= 1e-13


def test_lse_against_scalar_loops():
    q, k, v, dout, pos = case(5, 1, 7, 1, 16)
    _, _, _, lse = attention_backward(q, k, v, pos, dout)
    qr = rope4d(q, pos)[0, :, 0]
    kr = rope4d(k, pos)[0, :, 0]
    for i in range(7):
        s = [sum(qr[i, d] * kr[j, d] for d in range(16)) / 4.0 for j in range(7)]
        want = math.log(sum(math.exp(x) for x in s))
        assert abs(lse[0, 0, i] - want) <= 1e-12


# ------------------------------------------------------------ planted mistakes

def _mutants():
    """Plausible backward bugs, each a broken _backward_head."""
    good = bwd_mod._backward_head

    def plus_rotation(q, k, v, dout, pos, theta):
        # rotate the gradients back by +p (R instead of R^T)
        D = q.shape[-1]
        c = 1.0 / np.sqrt(D)
        qr = rope4d(q[:, None, :], pos, theta)[:, 0, :]
        kr = rope4d(k[:, None, :], pos, theta)[:, 0, :]
        s = (qr @ kr.T) * c
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        o = p @ v
        ds = p * (dout @ v.T - np.sum(dout * o, 1, keepdims=True))
        dq = rope4d(((ds @ kr) * c)[:, None, :], pos, theta)[:, 0, :]
        dk = rope4d(((ds.T @ qr) * c)[:, None, :], pos, theta)[:, 0, :]
        return dq, dk, p.T @ dout, np.zeros(q.shape[0])

    def no_delta(q, k, v, dout, pos, theta):
        dq, dk, dv, lse = good(q, k, v, np.zeros_like(dout), pos, theta)
        D = q.shape[-1]
        c = 1.0 / np.sqrt(D)
        qr = rope4d(q[:, None, :], pos, theta)[:, 0, :]
        kr = rope4d(k[:, None, :], pos, theta)[:, 0, :]
        s = (qr @ kr.T) * c
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        ds = p * (dout @ v.T)
        dq = rope4d(((ds @ kr) * c)[:, None, :], -pos, theta)[:, 0, :]
        dk = rope4d(((ds.T @ qr) * c)[:, None, :], -pos, theta)[:, 0, :]
        return dq, dk, p.T @ dout, lse

    def no_scale(q, k, v, dout, pos, theta):
        dq, dk, dv, lse = good(q, k, v, dout, pos, theta)
        return dq * np.sqrt(q.shape[-1]), dk, dv, lse

    def ds_not_transposed(q, k, v, dout, pos, theta):
        D = q.shape[-1]
        c = 1.0 / np.sqrt(D)
        qr = rope4d(q[:, None, :], pos, theta)[:, 0, :]
        kr = rope4d(k[:, None, :], pos, theta)[:, 0, :]
        s = (qr @ kr.T) * c
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        o = p @ v
        ds = p * (dout @ v.T - np.sum(dout * o, 1, keepdims=True))
        dq = rope4d(((ds @ kr) * c)[:, None, :], -pos, theta)[:, 0, :]
        dk = rope4d(((ds @ qr) * c)[:, None, :], -pos, theta)[:, 0, :]
        return dq, dk, p.T @ dout, np.zeros(q.shape[0])

    return [plus_rotation, no_delta, no_scale, ds_not_transposed]


def _fd_pin_passes():
    q, k, v, dout, pos = case(6, 1, 4, 1, 8)
    dq, dk, dv, _ = attention_backward(q, k, v, pos, dout, workers=1)
    fq, fk, fv = finite_differences(q, k, v, dout, pos)
    return all(np.max(np.abs(g - w)) <= 1e-7 * max(1.0, np.max(np.abs(w)))
               for g, w in ((dq, fq), (dk, fk), (dv, fv)))


def test_fd_pin_passes_on_good_oracle():
    assert _fd_pin_passes()


@pytest.mark.parametrize("i", range(4))
def test_planted_backward_mistake_is_caught(monkeypatch, i):
    monkeypatch.setattr(bwd_mod, "_backward_head", _mutants()[i])
    assert not _fd_pin_passes()
