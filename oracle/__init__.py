"""CPU float64 oracle for RoPE-4D joint self-attention -- TEST INFRASTRUCTURE.

This package is the reference the GPU path is tested against, not part of the
product.  Only the test suite, the smoke check of the entry module and the
CPU-baseline leg of the benchmark may import it.  It shares no code with the
HIP library: the only thing both sides consume is the seeded input generator
in ``workloads``, which holds none of the method's arithmetic.

What it computes, per batch entry b and head h (sources: "Flux.3 Image Klein
arrives in Diffusers with a modular architecture", bytechap.com, section "How
it works" -- joint blocks in which every token attends to every other token,
and a rotary embedding over the four axes time step, height, width and
sequence length; "FLUX.3 Image Klein open weights ...", kimiseek.app, section
"Limitations and unconfirmed points" -- one prompt per call and the prompt
padding is attended, so there is no mask):

  1. upcast the stored inputs exactly to float64 (bf16 bits, or e4m3 code times
     its per-tensor descale);
  2. rotate Q and K with RoPE-4D at each token's own (t, h, w, l) position;
  3. s_ij = <q'_i, k'_j> / sqrt(D) over all i, j (no mask, not causal);
  4. p_ij = softmax_j(s_ij);
  5. o_i = sum_j p_ij v_j.

Readings of points the pages leave open (each is also listed in the design
notes): theta = 10000 with the frequency schedule theta^(-2j/d_a) per axis;
D split into four equal blocks in the order t, h, w, l; rotation on
interleaved channel pairs (2j, 2j+1) as (x cos - y sin, x sin + y cos);
softmax scale 1/sqrt(D); positions shared by every batch entry.

Modules:
  rope4d     -- the rotary embedding (pinned: orthogonality, norm, identity at
                p = 0, relative-position property, brute force)
  joint_attention -- the attention definition above, plus exact storage decoders
                (pinned: brute force, scaled_dot_product_attention at p = 0,
                softmax invariants)
  brute      -- pure-Python scalar loops for tiny shapes (the brute-force pin)
  fp8        -- OCP E4M3FN decoding (pinned: all 256 codes against the
                format's definition and torch.float8_e4m3fn)
  qkv_proj   -- the QKV projection feeding the attention, with RoPE-4D on its
                q and k outputs (pinned: brute force, torch's linear at p = 0,
                composition with the attention)
  blocksparse -- the same attention restricted to kept (query block, key
                block) pairs, the reading of the pages' sparsified attention
                (pinned: brute force, every block kept = dense, one kept block
                = dense on that block's keys)
  backward   -- gradients of q, k, v through the attention and the rotation,
                and the softmax log-sum-exp (pinned: finite differences of the
                forward, torch autograd at p = 0, softmax invariants)
"""

from .joint_attention import (
    attention,
    attention_inputs_rows,
    attention_rows,
    bf16_to_f64,
    decode_inputs,
)
from .backward import attention_backward
from .blocksparse import (
    attention_blocksparse,
    attention_blocksparse_inputs_rows,
    attention_blocksparse_rows,
)
from .fp8 import e4m3_decode
from .qkv_proj import qkv_rope4d_proj
from .rope4d import rope4d, rope_frequencies

__all__ = [
    "attention",
    "attention_backward",
    "attention_blocksparse",
    "attention_blocksparse_inputs_rows",
    "attention_blocksparse_rows",
    "attention_inputs_rows",
    "attention_rows",
    "bf16_to_f64",
    "decode_inputs",
    "e4m3_decode",
    "qkv_rope4d_proj",
    "rope4d",
    "rope_frequencies",
]
