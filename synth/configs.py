"""Workload table for the canvas denoise step.

Every workload is a single-layer synthetic stand-in for the backbone that the
DiffusionGemma explainer names ("Architettura: il prefill incrementale e il
denoising"): a 256-token canvas (section on the autoregressive problem and the
"Campionamento multi-canvas" section) attending bidirectionally over a KV cache
plus itself, a tied vocabulary head, self-conditioning P.E and uniform-state
renoising below a confidence threshold ("Diffusione dello stato uniforme").
The pages print no sizes other than the 256-token canvas; the remaining
sizes are synthetic choices listed here with their purpose.
"""
from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class Config:
    name: str
    index: int            # used only to seed the generators
    B: int                # independent canvases
    C: int                # canvas length
    L: int                # KV-cache length at the start of block 0
    d: int                # model width
    Hq: int               # query heads
    Hkv: int              # key/value heads (GQA: Hq % Hkv == 0)
    dh: int               # head dim
    V: int                # vocabulary size
    dtype: str            # "f32" or "bf16" storage; accumulation is fp32 on the GPU
    steps: int            # denoise steps per block
    blocks: int           # canvases diffused one after another (block diffusion)
    tau: Tuple[float, float]  # (first, last) threshold; equal for a constant tau
    kv_std: float = -1.0  # std of cached K/V; <0 means 1/sqrt(d)
    purpose: str = field(default="", compare=False)

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def R(self):
        return self.B * self.C

    @property
    def cap(self):
        """Cache capacity: room for every finalized block appended after it is
        diffused (block diffusion appends each of the `blocks` canvases)."""
        return self.L + self.blocks * self.C if self.blocks > 1 else self.L

    @property
    def seed(self):
        """Philox key word 0 for this workload's token draws."""
        return 1000 + self.index

    @property
    def cache_std(self):
        return self.kv_std if self.kv_std > 0 else self.d ** -0.5


def tau_schedule(cfg: Config):
    """Threshold per denoise step of a block: linear from first to last, both
    endpoints included (constant when they are equal)."""
    a, b = cfg.tau
    if cfg.steps == 1 or a == b:
        return [float(a)] * cfg.steps
    return [a + (b - a) * s / (cfg.steps - 1) for s in range(cfg.steps)]


CONFIGS = [
    Config("tiny_c16_L32_d64_V512_f32", 0, B=1, C=16, L=32, d=64, Hq=2, Hkv=1, dh=32,
           V=512, dtype="f32", steps=4, blocks=1, tau=(0.5, 0.5),
           purpose="fp32 parity case small enough for the pure-Python brute force"),
    Config("canvas256_L1024_d2048_V32768", 1, B=1, C=256, L=1024, d=2048, Hq=16, Hkv=8,
           dh=128, V=32768, dtype="bf16", steps=8, blocks=1, tau=(0.9, 0.9),
           purpose="small-vocabulary bf16 step"),
    Config("canvas256_L8192_d2048_V262144", 2, B=1, C=256, L=8192, d=2048, Hq=16, Hkv=8,
           dh=128, V=262144, dtype="bf16", steps=16, blocks=1, tau=(0.9, 0.9),
           purpose="full-vocabulary step: the vocab/self-conditioning pass dominates"),
    Config("canvas256_L32768_d4096_V262144", 3, B=1, C=256, L=32768, d=4096, Hq=32, Hkv=8,
           dh=128, V=262144, dtype="bf16", steps=16, blocks=1, tau=(0.8, 0.8), kv_std=1.0,
           purpose="long cache, wide model"),
    Config("blocks4_canvas8x256_L4096_d2048_V262144", 4, B=8, C=256, L=4096, d=2048, Hq=16,
           Hkv=8, dh=128, V=262144, dtype="bf16", steps=32, blocks=4, tau=(0.5, 0.95),
           purpose="block diffusion: 8 canvases, 4 blocks, causal append after each block"),
]


def config_by_name(name_or_index):
    if isinstance(name_or_index, int):
        return CONFIGS[name_or_index]
    for c in CONFIGS:
        if c.name == name_or_index:
            return c
    raise KeyError(name_or_index)
