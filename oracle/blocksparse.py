"""Block-sparse joint attention with RoPE-4D in float64 -- oracle (test
infrastructure).

Source: "How FLUX 3 Image Klein was made 3-4x faster on NVIDIA Blackwell",
section "Method 2": one of the attention speed-ups leaves out the computation
of weakly related query/key combinations (sparsification), runs the early
denoising steps dense and only the later ones sparse.  The page gives no rule
for picking the combinations, so this reading takes them as an input: per
batch entry b and head h, a mask over blocks of QB consecutive queries by KB
consecutive keys; a query attends only to the keys of the kept blocks of its
query block:

    s_ij = <q'_i, k'_j> / sqrt(D)          (as in joint_attention)
    p_ij = exp(s_ij - m_i) / sum_{j kept} exp(s_ij - m_i),  m_i = max_{j kept} s_ij
    o_i  = sum_{j kept} p_ij v_j

for j in the kept blocks of block(i) only.  A query whose block keeps no key
block has o_i = 0 (an empty softmax).  With every block kept this is exactly
the dense definition.

Parity: pinned against a pure-Python scalar loop (oracle.brute), against the
dense oracle with every block kept, and against the dense oracle run on only
the keys of the single kept block.
"""

import numpy as np

from .joint_attention import ROW_BLOCK, _run, decode_inputs
from .rope4d import THETA, rope4d


def key_mask_rows(mask_bh, rows, S, qblock, kblock):
    """Boolean [len(rows), S]: key j is kept for query row r."""
    kb = np.arange(S) // kblock
    return mask_bh[rows // qblock][:, kb] != 0


def _attend_head_sparse(q, k, v, pos_q, pos_k, keep, theta):
    """One head: q [R, D], k, v [S, D]; keep [R, S] boolean."""
    D = q.shape[-1]
    qr = rope4d(q[:, None, :], pos_q, theta)[:, 0, :]
    kr = rope4d(k[:, None, :], pos_k, theta)[:, 0, :]
    s = (qr @ kr.T) / np.sqrt(D)
    s = np.where(keep, s, -np.inf)
    any_kept = keep.any(axis=1)
    m = np.where(any_kept, s.max(axis=1), 0.0)
    e = np.where(keep, np.exp(s - m[:, None]), 0.0)
    z = e.sum(axis=1)
    out = (e @ v) / np.where(any_kept, z, 1.0)[:, None]
    out[~any_kept] = 0.0
    return out


def attention_blocksparse_rows(q, k, v, pos, mask, rows, qblock, kblock,
                               theta: float = THETA, workers=None) -> np.ndarray:
    """Rows ``rows`` of every (b, h): float64 [B, len(rows), H, D].

    q, k, v float64 [B, S, H, D]; pos int [S, 4]; mask [B, H, ceil(S/qblock),
    ceil(S/kblock)] (nonzero = compute the block).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    B, S, H, D = q.shape
    mask = np.asarray(mask)
    if mask.shape != (B, H, -(-S // qblock), -(-S // kblock)):
        raise ValueError("mask must be [B, H, ceil(S/qblock), ceil(S/kblock)]")
    out = np.empty((B, rows.size, H, D), dtype=np.float64)

    def task(args):
        b, h, lo = args
        sel = rows[lo:lo + ROW_BLOCK]
        keep = key_mask_rows(mask[b, h], sel, S, qblock, kblock)
        out[b, lo:lo + sel.size, h] = _attend_head_sparse(
            q[b, sel, h], k[b, :, h], v[b, :, h], pos[sel], pos, keep, theta)

    _run(task, [(b, h, lo) for b in range(B) for h in range(H)
                for lo in range(0, rows.size, ROW_BLOCK)], workers)
    return out


def attention_blocksparse(q, k, v, pos, mask, qblock, kblock, theta: float = THETA,
                          workers=None) -> np.ndarray:
    """Full output [B, S, H, D] (float64)."""
    S = np.asarray(q).shape[1]
    return attention_blocksparse_rows(q, k, v, pos, mask, np.arange(S), qblock, kblock,
                                      theta, workers)


def attention_blocksparse_inputs_rows(inp, mask, rows, qblock, kblock, theta: float = THETA,
                                      workers=None) -> np.ndarray:
    """Like attention_blocksparse_rows, decoding one (b, h) slice of a
    workload's stored inputs (bf16 bits or e4m3 codes) at a time."""
    rows = np.asarray(rows, dtype=np.int64)
    B, S, H, D = inp.q.shape
    mask = np.asarray(mask)
    out = np.empty((B, rows.size, H, D), dtype=np.float64)

    def task(args):
        b, h = args
        qh, kh, vh = decode_inputs(inp, b, h)
        for lo in range(0, rows.size, ROW_BLOCK):
            sel = rows[lo:lo + ROW_BLOCK]
            keep = key_mask_rows(mask[b, h], sel, S, qblock, kblock)
            out[b, lo:lo + sel.size, h] = _attend_head_sparse(
                qh[sel], kh, vh, inp.pos[sel], inp.pos, keep, theta)

    _run(task, [(b, h) for b in range(B) for h in range(H)], workers)
    return out
