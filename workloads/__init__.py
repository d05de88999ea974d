"""Seeded synthetic inputs for RoPE-4D joint attention.

This package only *makes* inputs: token positions, bf16 Q/K/V bit patterns and
fp8-e4m3 codes with their per-tensor scales.  It holds none of the attention or
rotary arithmetic, so the HIP library and the CPU oracle can both consume the
exact same bits without sharing any of the method's code.

Token layout follows the joint sequence the FLUX.3 Image Klein pages describe
("Flux.3 Image Klein arrives in Diffusers with a modular architecture",
bytechap.com, section "How it works"; "FLUX.3 Image Klein open weights ...",
kimiseek.app, sections "Main changes" and "Adoption and evaluation
proposals"): text tokens first, laid out on the sequence-length axis l, then
the 16x16-pixel-patch latent grid of the image on (h, w), then each reference
image on the same (h, w) grid, told apart from the output by the t axis.
"""

from .configs import CONFIGS, Config, get_config
from .generate import (
    make_block_mask,
    Inputs,
    bf16_bits_from_f32,
    e4m3_encode,
    make_inputs,
    make_positions,
)

__all__ = [
    "make_block_mask",
    "CONFIGS",
    "Config",
    "Inputs",
    "bf16_bits_from_f32",
    "e4m3_encode",
    "get_config",
    "make_inputs",
    "make_positions",
]
