"""Joint self-attention with RoPE-4D in float64 -- oracle (test infrastructure).

Definition followed (sources: "Flux.3 Image Klein arrives in Diffusers with a
modular architecture", section "How it works": after the per-stream blocks the
text, image and reference tokens are concatenated and every token attends to
every other token, with the four-axis rotary embedding; "FLUX.3 Image Klein
open weights ...", section "Limitations and unconfirmed points": the prompt
padding is attended, so no key is masked; same page, section "Adoption and
evaluation proposals": reference and output share (h, w), so positions are per
token and the same for every batch entry):

    q'_i = RoPE(q_i, pos_i),  k'_j = RoPE(k_j, pos_j)
    s_ij = <q'_i, k'_j> / sqrt(D)                   for all i, j in [0, S)
    p_ij = exp(s_ij - max_j s_ij) / sum_j exp(s_ij - max_j s_ij)
    o_i  = sum_j p_ij v_j

independently for every batch entry b and head h.  Each output row depends only
on its own query, so computing rows in blocks (to bound memory) or in parallel
(to use the host cores) changes no arithmetic of any row.

Parity: pinned by tests against pure-Python brute force on tiny shapes, against
torch.nn.functional.scaled_dot_product_attention (float64, CPU) when every
position is zero (RoPE is then the identity), and against the softmax
invariants (V = 1 gives 1, equal keys give the mean of V, S = 1 gives V).
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .fp8 import e4m3_decode
from .rope4d import THETA, rope4d

ROW_BLOCK = 256


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 values of bfloat16 bit patterns (uint16)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode_inputs(inp, b=None, h=None):
    """float64 (q, k, v) of a workload, optionally only batch b / head h.

    ``inp`` carries uint16 bf16 patterns, or uint8 e4m3 codes plus per-tensor
    descales (value = decode(code) * descale).
    """
    def pick(x):
        if b is not None:
            x = x[b]
        if h is not None:
            x = x[..., h, :]
        return x

    out = []
    for i, x in enumerate((inp.q, inp.k, inp.v)):
        x = pick(x)
        if inp.descale is None:
            out.append(bf16_to_f64(x))
        else:
            out.append(e4m3_decode(x) * float(np.float32(inp.descale[i])))
    return tuple(out)


def _attend_head(q, k, v, pos_q, pos_k, theta):
    """One head: q [R, D] at positions pos_q [R, 4]; k, v [S, D] at pos_k."""
    D = q.shape[-1]
    qr = rope4d(q[:, None, :], pos_q, theta)[:, 0, :]
    kr = rope4d(k[:, None, :], pos_k, theta)[:, 0, :]
    s = (qr @ kr.T) / np.sqrt(D)                      # [R, S]
    s -= s.max(axis=1, keepdims=True)
    e = np.exp(s)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ v                                       # [R, D]


def _workers(workers):
    return workers or len(os.sched_getaffinity(0))


def attention(q, k, v, pos, theta: float = THETA, workers=None) -> np.ndarray:
    """Full output [B, S, H, D] (float64) from float64 q, k, v [B, S, H, D]."""
    q = np.asarray(q, dtype=np.float64)
    S = q.shape[1]
    return attention_rows(q, k, v, pos, np.arange(S), theta, workers)


def attention_rows(q, k, v, pos, rows, theta: float = THETA, workers=None) -> np.ndarray:
    """Output rows ``rows`` of every (b, h): float64 [B, len(rows), H, D].

    q, k, v: float64 [B, S, H, D]; pos: int [S, 4] shared across B.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    pos = np.asarray(pos)
    rows = np.asarray(rows, dtype=np.int64)
    B, S, H, D = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, S, H, D] shape")
    out = np.empty((B, rows.size, H, D), dtype=np.float64)

    def task(args):
        b, h, lo = args
        sel = rows[lo:lo + ROW_BLOCK]
        out[b, lo:lo + sel.size, h] = _attend_head(
            q[b, sel, h], k[b, :, h], v[b, :, h], pos[sel], pos, theta)

    jobs = [(b, h, lo) for b in range(B) for h in range(H)
            for lo in range(0, rows.size, ROW_BLOCK)]
    _run(task, jobs, workers)
    return out


def attention_inputs_rows(inp, rows, theta: float = THETA, workers=None) -> np.ndarray:
    """Like attention_rows, decoding one (b, h) slice of ``inp`` at a time."""
    rows = np.asarray(rows, dtype=np.int64)
    B, S, H, D = inp.q.shape
    out = np.empty((B, rows.size, H, D), dtype=np.float64)

    def task(args):
        b, h = args
        qh, kh, vh = decode_inputs(inp, b, h)
        for lo in range(0, rows.size, ROW_BLOCK):
            sel = rows[lo:lo + ROW_BLOCK]
            out[b, lo:lo + sel.size, h] = _attend_head(
                qh[sel], kh, vh, inp.pos[sel], inp.pos, theta)

    _run(task, [(b, h) for b in range(B) for h in range(H)], workers)
    return out


def _run(task, jobs, workers):
    """Run independent per-row-block jobs on ``workers`` threads.

    NumPy releases the GIL inside BLAS and ufuncs; BLAS itself is held to one
    thread per worker so the pool, not BLAS, spreads work over the cores.
    """
    from threadpoolctl import threadpool_limits
    n = _workers(workers)
    with threadpool_limits(limits=1):
        if n <= 1 or len(jobs) <= 1:
            for j in jobs:
                task(j)
        else:
            with ThreadPoolExecutor(max_workers=n) as ex:
                list(ex.map(task, jobs))
