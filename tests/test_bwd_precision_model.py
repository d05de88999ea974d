"""A CPU model of the attention backward's roundings (CPU only).

The backward kernels feed ds = p (dp - delta) to their MFMAs as fp16, whose
normal range (2^-14 .. 65504) is much narrower than fp32's.  This models one
head of the GPU backward step by step in NumPy -- fp16 rotated operands, P
from exp2 of the fp32 scores, ds rounded to fp16, gradients accumulated in
float64 and rounded once to bf16 -- and compares it with the float64 oracle:

* with ds rounded as it is (no scale), gradients of the size fine-tuning
  produces (|dout| ~ 1e-4 and below) push ds into fp16's subnormals and to
  zero, and dq, dk miss the 6e-3 relative-L2 bound; large gradients overflow
  fp16 to inf;
* with the power-of-two scale 2^e the kernels apply (e = 14 - ceil(log2(2
  max_i |dout_i| max_j |v_j|)), added to the scores' exponent and removed
  exactly at the end) the error is the same at every gradient size, and the
  largest |2^e ds| stays below 2^14.

The model is test code: it restates the kernel's rounding steps, not its
arithmetic order, and is not used by any GPU test.
"""

import numpy as np
import pytest

import oracle
from workloads import bf16_bits_from_f32

GRAD_REL_L2 = 6e-3
LOG2E = 1.0 / np.log(2.0)


def bf16(x):
    bits = bf16_bits_from_f32(np.asarray(x, dtype=np.float32))
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f16(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def scale_exponent(dout, v):
    """The kernels' rule: 2^e times the bound 2 max|dout_i| max|v_j| stays below 2^14."""
    bound = 2.0 * np.sqrt(np.max(np.sum(dout * dout, axis=1))) * \
        np.sqrt(np.max(np.sum(v * v, axis=1))) * (1.0 + 1.0 / 256.0)
    if bound == 0.0:
        return 14
    _, ex = np.frexp(bound)
    return int(np.clip(14 - ex, -100, 100))


def model_backward(q, k, v, dout, pos, e):
    """(dq, dk, dv, max |2^e ds|) of one head, [S, D] each, the way the
    kernels round them, with scale exponent e."""
    S, D = q.shape
    qr = oracle.rope4d(q[:, None, :], pos)[:, 0, :]
    kr = oracle.rope4d(k[:, None, :], pos)[:, 0, :]
    q2 = f16(qr * LOG2E / np.sqrt(D))                 # q'' (fp16)
    k2 = f16(kr)                                      # k' (fp16)
    s2 = q2 @ k2.T                                    # exp2-domain scores
    m = s2.max(axis=1, keepdims=True)
    lse2 = m + np.log2(np.exp2(s2 - m).sum(axis=1, keepdims=True))
    p = np.exp2(s2 - lse2 + e)                        # 2^e p (fp32 in the kernel)
    out = bf16(np.exp2(s2 - lse2) @ v)                # the forward's bf16 output
    delta = np.sum(dout * out, axis=1, keepdims=True)
    dp = dout @ v.T
    ds = f16(p * (dp - delta))                        # fp16 MFMA operand
    dv = bf16((bf16(p).T @ dout) * 2.0 ** -e)
    dkr = (ds.T @ q2) * 2.0 ** -e / LOG2E
    dqr = (ds @ k2) * 2.0 ** -e / np.sqrt(D)
    back = lambda x: oracle.rope4d(x[:, None, :], -pos)[:, 0, :]
    with np.errstate(invalid="ignore"):
        return bf16(back(dqr)), bf16(back(dkr)), dv, float(np.max(np.abs(ds)))


@pytest.fixture(scope="module")
def head():
    rng = np.random.default_rng(11)
    S, D = 768, 128
    q, k, v = (bf16(rng.standard_normal((S, D))) for _ in range(3))
    g = rng.standard_normal((S, D))
    pos = rng.integers(-50, 600, size=(S, 4)).astype(np.int32)
    return q, k, v, g, pos


def rel_errors(model, ref):
    out = []
    for a, r in zip(model, ref):
        if not np.isfinite(a).all():
            out.append(np.inf)
        else:
            out.append(float(np.linalg.norm(a - r) / np.linalg.norm(r)))
    return out


@pytest.mark.parametrize("gscale", [1.0, 1e-4, 1e-6, 1e-12, 1e5])
def test_scaled_ds_meets_the_bound_at_every_gradient_size(head, gscale):
    q, k, v, g, pos = head
    dout = bf16(g * gscale)
    ref = oracle.attention_backward(q[None, :, None], k[None, :, None], v[None, :, None],
                                    pos, dout[None, :, None])
    ref = [r[0, :, 0] for r in ref[:3]]
    e = scale_exponent(dout, v)
    *grads, ds_max = model_backward(q, k, v, dout, pos, e)
    errs = rel_errors(grads, ref)
    print(f"scale {gscale:g}: e = {e}, max |2^e ds| = {ds_max:.3g}, rel-L2 dq dk dv = "
          + " ".join(f"{x:.2e}" for x in errs))
    assert ds_max < 2.0 ** 14
    assert max(errs) <= 0.5 * GRAD_REL_L2, (gscale, e, errs)


@pytest.mark.parametrize("gscale", [1e-4, 1e-6])
def test_unscaled_fp16_ds_fails_on_small_gradients(head, gscale):
    q, k, v, g, pos = head
    dout = bf16(g * gscale)
    ref = oracle.attention_backward(q[None, :, None], k[None, :, None], v[None, :, None],
                                    pos, dout[None, :, None])
    ref = [r[0, :, 0] for r in ref[:3]]
    errs = rel_errors(model_backward(q, k, v, dout, pos, 0)[:3], ref)
    print(f"scale {gscale:g}, unscaled: rel-L2 dq dk dv = " + " ".join(f"{x:.2e}" for x in errs))
    assert errs[0] > GRAD_REL_L2 and errs[1] > GRAD_REL_L2, errs    # dq, dk
    assert errs[2] <= GRAD_REL_L2                                    # dv has no ds


def test_unscaled_fp16_ds_overflows_on_large_gradients(head):
    q, k, v, g, pos = head
    dout = bf16(g * 1e5)
    dq, dk, _, ds_max = model_backward(q, k, v, dout, pos, 0)
    assert not np.isfinite(ds_max) or not np.isfinite(dq).all() or not np.isfinite(dk).all()


def test_scale_rule_bounds_ds_for_adversarial_rows():
    # the bound holds for every row pair, not only on average: a dout row
    # parallel to a v row, with p concentrated on that key
    D = 128
    v = np.zeros((4, D))
    v[0] = 3.0
    dout = np.zeros((4, D))
    dout[1] = -5.0
    e = scale_exponent(dout, v)
    # |dp - delta| <= |dout_i| (|v_j| + max_j |v_j|) = 2 |dout_i| max |v_j|
    worst = 2 * np.linalg.norm(dout[1]) * np.linalg.norm(v[0])
    assert worst * 2.0 ** e < 2.0 ** 14 <= 2 * worst * 2.0 ** e * (1 + 1 / 256)
    assert scale_exponent(np.zeros((4, D)), v) == 14
