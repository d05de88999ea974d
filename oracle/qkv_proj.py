"""QKV projection with the RoPE-4D rotation applied to its output, in float64
-- oracle (test infrastructure).

This is the step that feeds the attention ("Flux.3 Image Klein arrives in
Diffusers with a modular architecture", section "How it works": each joint
block projects the concatenated token sequence to queries, keys and values
and rotates queries and keys with the four-axis rotary embedding; "How FLUX 3
Image Klein was made 3-4x faster on NVIDIA Blackwell", section "Method 1":
the QKV projections are fused GEMMs).  With x [B, S, C], a weight W
[3 H D, C] (a linear layer's [out, in] layout) and an optional bias [3 H D]:

    y = x W^T + bias                        [B, S, 3 H D]
    q, k, v = y[..., :HD], y[..., HD:2HD], y[..., 2HD:]   each [B, S, H, D]
    q' = RoPE-4D(q, pos),  k' = RoPE-4D(k, pos),  v unrotated

Attention of (q', k', v) without a rotation is then exactly the fused
definition of joint_attention on (q, k, v, pos).

Parity: pinned against pure-Python scalar loops, against
torch.nn.functional.linear (float64) when every position is zero, and by the
composition with the attention oracle.
"""

import numpy as np

from .rope4d import THETA, rope4d


def qkv_rope4d_proj(x, w, bias, pos, H, D, theta: float = THETA):
    """(q', k', v), each float64 [B, S, H, D]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, S, C = x.shape
    if w.shape != (3 * H * D, C):
        raise ValueError("w must be [3 H D, C]")
    y = x @ w.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)
    y = y.reshape(B, S, 3, H, D)
    q, k, v = y[:, :, 0], y[:, :, 1], y[:, :, 2]
    return rope4d(q, pos, theta), rope4d(k, pos, theta), v.copy()
