"""A NumPy model of the FP8 attention kernel's roundings (test code, CPU only).

It restates, step by step, what the fp8 kernel computes for one head, so that
its precision choices can be priced against the float64 oracle on the CPU:

  Q'' = e4m3(R(q_code) c)                  rotated in fp32, c = G / 2^n
  K'' = e4m3(R(k_code) / 2)                rotated in packed fp16
  Y   = 8 (s2 - m) + ym                    s2 the exp2-domain score, m the
                                           running row max (in Y units, m8)
  P8  = the E4M3 code rne(clamp(Y, 0, 255)), read as a number
  O  += V_code P8,  l += sum P8,  out = bf16(O dv / l)

The running max starts at the exact row max of the first 64-key tile.  A wave
of 32 queries checks each tile's row maxima; when any of its rows has a code
above 126 (E4M3's largest finite value, 448), every row of the wave moves its
max to code ym_post where its tile max lies higher (delta = max(Ymax -
ym_post, 0)), and O and l are scaled by 2^(-delta/8).  Codes below 0.5 round
to 0: a key more than about (ym + 0.5)/8 binades below the first running
max, or (ym_post + 0.5)/8 below a raised one, contributes nothing.  The
kernel's values: ym = 118, ym_post = 110.  The split-KV schedule's chunks follow the same
rules from their own first tile; this model covers the whole-tile path.
"""

import numpy as np

import oracle
from workloads import e4m3_encode

LOG2E = 1.0 / np.log(2.0)
BN = 64          # keys per tile
WAVE = 32        # queries per wave
YMAX = 126.0     # code of 448


def f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def bf16(x):
    x = np.asarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3(x):
    return oracle.e4m3_decode(e4m3_encode(x))


def score_split(descale, D):
    """G = 2 dq dk log2(e) / sqrt(D) = c 2^n with c in (1/(2 sqrt 2), 1/sqrt 2]."""
    G = descale[0] * descale[1] * LOG2E * 2.0 / np.sqrt(D)
    n = int(np.ceil(np.log2(G * np.sqrt(2.0))))
    return G / 2.0 ** n, n


def angles(pos, D):
    """phi[s, c/2]: the rotation angle of channel pair c/2 at token s."""
    da = D // 4
    j = np.arange(da // 2)
    w = 10000.0 ** (-2.0 * j / da)
    return np.concatenate([pos[:, a:a + 1] * w[None, :] for a in range(4)], axis=1)


def rotate_q(qc, pos, c):
    """Q'' = e4m3(R(q_code) c), fp32 rotation."""
    phi = angles(pos, qc.shape[-1])
    x, y = qc[:, 0::2], qc[:, 1::2]
    cs, sn = np.cos(phi) * c, np.sin(phi) * c
    out = np.empty_like(qc)
    out[:, 0::2] = e4m3(x * cs - y * sn)
    out[:, 1::2] = e4m3(x * sn + y * cs)
    return out


def rotate_k(kc, pos):
    """K'' = e4m3(R(k_code) / 2) in packed fp16: (cos, sin)/2 held in fp16, y s and
    y c rounded to fp16, then one fp16 fma each."""
    phi = angles(pos, kc.shape[-1])
    x, y = kc[:, 0::2], kc[:, 1::2]
    cs, sn = f16(np.cos(phi) * 0.5), f16(np.sin(phi) * 0.5)
    out = np.empty_like(kc)
    out[:, 0::2] = e4m3(f16(x * cs - f16(y * sn)))
    out[:, 1::2] = e4m3(f16(x * sn + f16(y * cs)))
    return out


def attention_head(qc, kc, vc, pos, descale, rows, ym=118.0, stats=None, ym_post=110.0):
    """Output rows ``rows`` of one head (float64 values of the bf16 result).

    qc, kc, vc: float64 E4M3 code values [S, D] (no descale); every wave that
    holds one of ``rows`` is modelled in full (its rescale decisions depend
    on all 32 of its queries).  ``stats`` (a dict), if given, receives the
    number of rescales per wave and tile.  ``ym_post``: the code a rescale
    moves a row's max to (None: ym)."""
    ym_post = ym if ym_post is None else ym_post
    S, D = qc.shape
    c, n = score_split(descale, D)
    waves = np.unique(np.asarray(rows) // WAVE)
    qidx = (waves[:, None] * WAVE + np.arange(WAVE)[None, :]).clip(max=S - 1)   # [W, 32]
    q2 = rotate_q(qc, pos, c)[qidx]                                            # [W, 32, D]
    k2 = rotate_k(kc, pos)
    nkt = -(-S // BN)
    scale = 2.0 ** (n + 3)
    W = waves.size
    o = np.zeros((W, WAVE, D))
    lsum = np.zeros((W, WAVE))
    m8 = np.zeros((W, WAVE))
    rescales = 0
    for t in range(nkt):
        k0, k1 = t * BN, min(S, t * BN + BN)
        raw = scale * np.einsum("wqd,kd->wqk", q2, k2[k0:k1])              # 8 s2
        if t == 0:
            m8 = raw.max(axis=2)
        y = raw - m8[..., None] + ym
        mx = y.max(axis=2)
        hit = (mx > YMAX).any(axis=1)                                        # per wave
        if hit.any():
            delta = np.where(hit[:, None], np.maximum(mx - ym_post, 0.0), 0.0)
            alpha = np.exp2(-delta / 8.0)
            m8 += delta
            o *= alpha[..., None]
            lsum *= alpha
            y -= delta[..., None]
            rescales += int(hit.sum())
        p8 = oracle.e4m3_decode(np.rint(np.clip(y, 0.0, 255.0)).astype(np.uint8))
        o += np.einsum("wqk,kd->wqd", p8, vc[k0:k1])
        lsum += p8.sum(axis=2)
    if stats is not None:
        stats["rescales_per_wave_tile"] = rescales / (W * nkt)
    out = bf16(o * descale[2] / lsum[..., None])                            # [W, 32, D]
    where = {int(w): i for i, w in enumerate(waves)}
    return np.stack([out[where[r // WAVE], r % WAVE] for r in rows])


def decode_codes(inp, b, h):
    """E4M3 code values (no descale) of one (b, h) slice of fp8 inputs."""
    return tuple(oracle.e4m3_decode(x[b, :, h, :]) for x in (inp.q, inp.k, inp.v))
