"""RoPE-4D in float64 -- oracle (test infrastructure only).

The pages say Klein's rotary position embedding runs over four axes -- time
step t, height h, width w and sequence length l -- with text tokens placed
along l and image/reference tokens on (h, w) ("Flux.3 Image Klein arrives in
Diffusers with a modular architecture", section "How it works").  They do not
print the formula, so this module takes the plainest reading that the rest
supports:

* the head dimension D is split into four equal blocks of d_a = D/4 channels,
  in the axis order t, h, w, l;
* inside axis block a (channel offset c_a = a * d_a), channel pair
  (c_a + 2j, c_a + 2j + 1), j = 0 .. d_a/2 - 1, is rotated by the angle
  phi = p_a * omega_j, omega_j = theta^(-2j / d_a), theta = 10000;
* a pair (x, y) becomes (x cos phi - y sin phi, x sin phi + y cos phi).

Parity: pinned by tests against closed forms (each pair is a 2x2 rotation, so
norms are kept and p = 0 is the identity), the relative-position property
<R(p) q, R(p') k> = <R(p + c) q, R(p' + c) k>, and pure-Python brute force.
"""

import numpy as np

THETA = 10000.0


def rope_frequencies(D: int, theta: float = THETA) -> np.ndarray:
    """omega_j = theta^(-2j/d_a) for j = 0 .. d_a/2 - 1, d_a = D/4 (float64)."""
    if D % 8 != 0:
        raise ValueError("RoPE-4D needs D divisible by 8 (four blocks of pairs)")
    da = D // 4
    j = np.arange(da // 2, dtype=np.float64)
    return theta ** (-2.0 * j / da)


def rope4d(x: np.ndarray, pos: np.ndarray, theta: float = THETA) -> np.ndarray:
    """Rotate x[..., S, H, D] (float64) by per-token positions pos[S, 4].

    Returns a new float64 array; the input is not modified.
    """
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(pos)
    S, H, D = x.shape[-3], x.shape[-2], x.shape[-1]
    if pos.shape != (S, 4):
        raise ValueError(f"pos must be [S, 4] = [{S}, 4], got {pos.shape}")
    da = D // 4
    omega = rope_frequencies(D, theta)               # [da/2]
    y = x.copy()
    for a in range(4):
        c = a * da
        phi = pos[:, a].astype(np.float64)[:, None] * omega[None, :]   # [S, da/2]
        cos = np.cos(phi)[:, None, :]                # broadcast over heads
        sin = np.sin(phi)[:, None, :]
        xe = x[..., c:c + da:2]                      # channels c + 2j
        xo = x[..., c + 1:c + da:2]                  # channels c + 2j + 1
        y[..., c:c + da:2] = xe * cos - xo * sin
        y[..., c + 1:c + da:2] = xe * sin + xo * cos
    return y
