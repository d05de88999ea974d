"""Backward of the RoPE-4D joint attention in float64 -- oracle (test infrastructure).

The pages ship training resources with the model: LoRA training scripts, and
DreamBooth-style training of instruction-based editing from (reference image,
target image, instruction) triples, with gradient checkpointing among the
memory options ("Flux.3 Image Klein arrives in Diffusers with a modular
architecture", sections "What happened" and "Key details").  Training runs the
joint attention backward: the gradients of a loss with respect to q, k and v,
through the rotary embedding, given the gradient dout of the attention output.

With the forward of joint_attention (per batch entry and head, R_i the RoPE-4D
rotation at token i's position, c = 1/sqrt(D)):

    q'_i = R_i q_i,  k'_j = R_j k_j,  s_ij = c <q'_i, k'_j>,
    p_ij = softmax_j(s_ij),  o_i = sum_j p_ij v_j

the chain rule gives, for a loss with dL/do_i = dout_i:

    dv_j   = sum_i p_ij dout_i
    dp_ij  = <dout_i, v_j>
    ds_ij  = p_ij (dp_ij - delta_i),   delta_i = <dout_i, o_i> = sum_j p_ij dp_ij
    dq'_i  = c sum_j ds_ij k'_j,       dk'_j = c sum_i ds_ij q'_i
    dq_i   = R_i^T dq'_i,              dk_j  = R_j^T dk'_j

and R^T at position p is the rotation at -p (each channel pair turns by an
angle linear in p, and a 2x2 rotation's transpose turns by minus that angle).

Parity: pinned by tests against central finite differences of the forward
oracle (an independent code path), against torch.autograd through
torch.nn.functional.scaled_dot_product_attention (float64) when every position
is zero, and against invariants: sum_j dv_j = sum_i dout_i (rows of p sum to
1); sum_j R_j dk_j = 0 and every dq_i = 0 when v is the same for every key
(softmax is unchanged by a shift of a row's scores).
"""

import numpy as np

from .joint_attention import _run
from .rope4d import THETA, rope4d


def _backward_head(q, k, v, dout, pos, theta):
    """One head, all rows: q, k, v, dout [S, D] -> (dq, dk, dv, lse) float64.

    lse_i = log sum_j exp(s_ij) (natural log), the softmax statistic a
    forward pass can hand to the backward."""
    D = q.shape[-1]
    c = 1.0 / np.sqrt(D)
    qr = rope4d(q[:, None, :], pos, theta)[:, 0, :]
    kr = rope4d(k[:, None, :], pos, theta)[:, 0, :]
    s = (qr @ kr.T) * c
    mx = s.max(axis=1, keepdims=True)
    e = np.exp(s - mx)
    den = e.sum(axis=1, keepdims=True)
    p = e / den
    lse = (mx + np.log(den))[:, 0]
    o = p @ v
    dv = p.T @ dout
    dp = dout @ v.T
    delta = np.sum(dout * o, axis=1, keepdims=True)
    ds = p * (dp - delta)
    dqr = (ds @ kr) * c
    dkr = (ds.T @ qr) * c
    dq = rope4d(dqr[:, None, :], -np.asarray(pos), theta)[:, 0, :]
    dk = rope4d(dkr[:, None, :], -np.asarray(pos), theta)[:, 0, :]
    return dq, dk, dv, lse


def attention_backward(q, k, v, pos, dout, theta: float = THETA, workers=None):
    """(dq, dk, dv) float64 [B, S, H, D] and lse float64 [B, H, S].

    q, k, v, dout: float64 [B, S, H, D]; pos: int [S, 4] shared across B.
    """
    q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    pos = np.asarray(pos)
    B, S, H, D = q.shape
    for x in (k, v, dout):
        if x.shape != q.shape:
            raise ValueError("q, k, v, dout must share one [B, S, H, D] shape")
    dq, dk, dv = (np.empty_like(q) for _ in range(3))
    lse = np.empty((B, H, S), dtype=np.float64)

    def task(args):
        b, h = args
        r = _backward_head(q[b, :, h], k[b, :, h], v[b, :, h], dout[b, :, h], pos, theta)
        dq[b, :, h], dk[b, :, h], dv[b, :, h], lse[b, h] = r

    _run(task, [(b, h) for b in range(B) for h in range(H)], workers)
    return dq, dk, dv, lse
