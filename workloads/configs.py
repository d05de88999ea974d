"""The five workload shapes of the RoPE-4D joint-attention hot path.

Token counts come from the pages: a 1024x1024 image is a 64x64 grid of 16x16
patches (4,096 tokens) and each 1024x1024 reference image adds another 4,096
tokens ("Flux.3 Image Klein arrives in Diffusers with a modular architecture",
section "How it works"; "FLUX.3 Image Klein open weights ...", section "Main
changes").  A 2048x2048 image is therefore a 128x128 grid (16,384 tokens).
Classifier-free guidance runs the model with and without the prompt ("How FLUX 3
Image Klein was made 3-4x faster on NVIDIA Blackwell", section "Premise 1"),
which is the B=2 batch of the CFG workload.
"""

from dataclasses import dataclass, field
from typing import Optional


@dataclass(frozen=True)
class Config:
    cid: int                 # workload number, also the seed base (1000 * cid)
    name: str
    B: int
    H: int
    D: int
    text: int                # text tokens, l = 0 .. text-1
    grid: int                # image latent grid side (grid x grid tokens)
    refs: int                # reference images, t = 1 .. refs, same grid
    dtype: str               # "bf16" or "fp8"
    prescale: bool = False   # multiply Q, K, V by 1/sqrt(D) at generation
    outliers: bool = False   # 1% of the H*D key channels scaled by 8
    uncond_zero_text: bool = False  # batch 1 (uncond): text-token Q/K/V = 0
    theta: float = 10000.0
    note: str = ""

    @property
    def S(self) -> int:
        return self.text + (1 + self.refs) * self.grid * self.grid

    @property
    def flops(self) -> int:
        """Attention flop count 4*B*H*S^2*D (QK^T and PV, 2 flops per MAC)."""
        return 4 * self.B * self.H * self.S * self.S * self.D


CONFIGS = {
    1: Config(1, "tiny", B=1, H=2, D=64, text=16, grid=8, refs=0, dtype="bf16",
              note="16 text + 8x8 image = 80 tokens"),
    2: Config(2, "1024px-t2i", B=1, H=24, D=128, text=512, grid=64, refs=0,
              dtype="bf16", prescale=True, outliers=True,
              note="512 text + 64x64 image = 4,608 tokens"),
    3: Config(3, "1024px-edit", B=1, H=24, D=128, text=512, grid=64, refs=1,
              dtype="bf16", outliers=True,
              note="512 text + 64x64 image + 64x64 reference = 8,704 tokens"),
    4: Config(4, "2048px-t2i-cfg", B=2, H=24, D=128, text=512, grid=128,
              refs=0, dtype="bf16", uncond_zero_text=True,
              note="512 text + 128x128 image = 16,896 tokens, cond+uncond"),
    5: Config(5, "2048px-edit-fp8", B=1, H=24, D=128, text=512, grid=128,
              refs=1, dtype="fp8",
              note="512 text + 128x128 image + 128x128 reference = 33,280 tokens"),
}


def get_config(cid: int, **overrides) -> Config:
    """Return workload ``cid``; keyword overrides build ragged/edge variants."""
    base = CONFIGS[cid]
    if not overrides:
        return base
    d = {f: getattr(base, f) for f in base.__dataclass_fields__}
    d.update(overrides)
    return Config(**d)
