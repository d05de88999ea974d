"""Pure-Python scalar RoPE-4D attention for tiny shapes -- brute-force pin.

Test infrastructure only.  Every quantity is a Python float computed one
scalar at a time with the math module, straight from the definition (see the
package docstring): rotate each interleaved channel pair of each axis block by
p_a * theta^(-2j/d_a), take all-pairs scaled dot products, softmax over keys,
weight the values.  No NumPy, no vectorisation, no blocking -- so it shares no
code path with the vectorised oracle it checks.
"""

import math


def rope_scalar(vec, p, theta=10000.0):
    """Rotate one D-vector (list of floats) at position p = (t, h, w, l)."""
    D = len(vec)
    da = D // 4
    out = list(vec)
    for a in range(4):
        for j in range(da // 2):
            ang = p[a] * theta ** (-2.0 * j / da)
            c, s = math.cos(ang), math.sin(ang)
            i0 = a * da + 2 * j
            x, y = vec[i0], vec[i0 + 1]
            out[i0] = x * c - y * s
            out[i0 + 1] = x * s + y * c
    return out


def attention_scalar(q, k, v, pos, theta=10000.0):
    """q, k, v: nested lists [B][S][H][D] of floats; pos: [S][4] ints."""
    B, S, H, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    out = [[[[0.0] * D for _ in range(H)] for _ in range(S)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            qr = [rope_scalar(q[b][i][h], pos[i], theta) for i in range(S)]
            kr = [rope_scalar(k[b][j][h], pos[j], theta) for j in range(S)]
            for i in range(S):
                s = [sum(qr[i][d] * kr[j][d] for d in range(D)) / math.sqrt(D)
                     for j in range(S)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = sum(e)
                for d in range(D):
                    out[b][i][h][d] = sum(e[j] * v[b][j][h][d] for j in range(S)) / z
    return out


def attention_blocksparse_scalar(q, k, v, pos, mask, qblock, kblock, theta=10000.0):
    """Block-sparse variant: query i attends to key j only when
    mask[b][h][i // qblock][j // kblock] is nonzero; no kept key gives 0."""
    B, S, H, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    out = [[[[0.0] * D for _ in range(H)] for _ in range(S)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            qr = [rope_scalar(q[b][i][h], pos[i], theta) for i in range(S)]
            kr = [rope_scalar(k[b][j][h], pos[j], theta) for j in range(S)]
            for i in range(S):
                kept = [j for j in range(S) if mask[b][h][i // qblock][j // kblock]]
                if not kept:
                    continue
                s = {j: sum(qr[i][d] * kr[j][d] for d in range(D)) / math.sqrt(D) for j in kept}
                m = max(s.values())
                e = {j: math.exp(s[j] - m) for j in kept}
                z = sum(e.values())
                for d in range(D):
                    out[b][i][h][d] = sum(e[j] * v[b][j][h][d] for j in kept) / z
    return out


def qkv_proj_scalar(x, w, bias, pos, H, D, theta=10000.0):
    """QKV projection then RoPE-4D on q and k, one scalar at a time.
    x: [B][S][C]; w: [3HD][C]; bias: [3HD] or None.  Returns q', k', v as
    nested lists [B][S][H][D]."""
    B, S, C = len(x), len(x[0]), len(x[0][0])
    outs = ([], [], [])
    for b in range(B):
        qb, kb, vb = [], [], []
        for s in range(S):
            y = [sum(x[b][s][c] * w[n][c] for c in range(C)) + (bias[n] if bias else 0.0)
                 for n in range(3 * H * D)]
            heads = [[y[t * H * D + h * D:t * H * D + (h + 1) * D] for h in range(H)]
                     for t in range(3)]
            qb.append([rope_scalar(heads[0][h], pos[s], theta) for h in range(H)])
            kb.append([rope_scalar(heads[1][h], pos[s], theta) for h in range(H)])
            vb.append([list(heads[2][h]) for h in range(H)])
        outs[0].append(qb); outs[1].append(kb); outs[2].append(vb)
    return outs
