"""Seeded synthetic inputs for the token-mixer layer shapes.

This module only draws random numbers and names shapes; it holds none of the
method's arithmetic.  Both the fp64 oracle (tests, CPU baseline) and the HIP
path (tests, bench, smoke) take their inputs from here.

Shapes follow "SANA-Video 2.0" (NVlabs Sana docs): section Architecture gives
20 heads x 128 for the 5B model and 32 heads x 128 for the 14B model, (1,1,1)
latent patches and (8, 32, 32) VAE strides; frame counts satisfy
(F - 1) % 8 == 0 (section Inference), so F frames give (F - 1)/8 + 1 latent
frames.  B = 2 is the classifier-free-guidance pair.

Recipe: a CPU ``torch.Generator`` seeded with the workload's seed draws fp32
N(0, 1) tensors of shape [B, N, H, D] in the order q, k, v, g; q and k are
multiplied by ``qk_scale`` (0.5 for the 14B shape); each is then rounded to
bf16 (round-to-nearest-even).  The data are iid with no structure: no real
projected video latents are available, so iid normals stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    D: int
    T: int   # latent frames
    Hh: int  # latent rows
    W: int   # latent columns
    qk_scale: float
    seed: int
    theta: float = 10000.0
    C: int = 0      # hidden size of the projection workloads (0: mixer inputs only)

    @property
    def N(self) -> int:
        return self.T * self.Hh * self.W

    @property
    def shape(self):
        return (self.B, self.N, self.H, self.D)

    def tensor_bytes(self) -> int:
        return self.B * self.N * self.H * self.D * 2


WORKLOADS = [
    Workload("tiny_d32_4x8x8", B=1, H=2, D=32, T=4, Hh=8, W=8, qk_scale=1.0, seed=0),
    Workload("5b_480p_81f", B=1, H=20, D=128, T=11, Hh=15, W=26, qk_scale=1.0, seed=1),
    Workload("5b_720p_193f", B=2, H=20, D=128, T=25, Hh=22, W=40, qk_scale=1.0, seed=2),
    Workload("14b_480p_193f", B=2, H=32, D=128, T=25, Hh=15, W=26, qk_scale=0.5, seed=3),
    Workload("5b_720p_60s", B=1, H=20, D=128, T=181, Hh=22, W=40, qk_scale=1.0, seed=4),
]
# The gated softmax anchor layers of the same models: 10 heads x 256 (5B) and
# 16 heads x 256 (14B) (section Architecture), on the same latent grids.
ANCHOR_WORKLOADS = [
    Workload("anchor_5b_480p_81f", B=1, H=10, D=256, T=11, Hh=15, W=26, qk_scale=1.0, seed=11),
    Workload("anchor_5b_720p_193f", B=2, H=10, D=256, T=25, Hh=22, W=40, qk_scale=1.0, seed=12),
    Workload("anchor_14b_480p_193f", B=2, H=16, D=256, T=25, Hh=15, W=26, qk_scale=1.0, seed=13),
]
# The projection prologue of the linear layers: hidden states x [B, N, C]
# with C = 2,560 (5B) or 4,096 (14B) (section Architecture) and the four
# stacked maps q, k, v, g of shape [4, H*D, C].
PROJ_WORKLOADS = [
    Workload("proj_tiny_d32_4x8x8", B=1, H=2, D=32, T=4, Hh=8, W=8, qk_scale=1.0, seed=20, C=128),
    Workload("proj_5b_480p_81f", B=1, H=20, D=128, T=11, Hh=15, W=26, qk_scale=1.0, seed=21,
             C=2560),
    Workload("proj_5b_720p_193f", B=2, H=20, D=128, T=25, Hh=22, W=40, qk_scale=1.0, seed=22,
             C=2560),
    Workload("proj_14b_480p_193f", B=2, H=32, D=128, T=25, Hh=15, W=26, qk_scale=1.0, seed=23,
             C=4096),
    Workload("proj_5b_720p_60s", B=1, H=20, D=128, T=181, Hh=22, W=40, qk_scale=1.0, seed=24,
             C=2560),
]
BY_NAME = {w.name: w for w in WORKLOADS + ANCHOR_WORKLOADS + PROJ_WORKLOADS}


def random_inputs(B: int, N: int, H: int, D: int, seed: int, qk_scale: float = 1.0):
    """(q, k, v, g): bf16 CPU tensors [B, N, H, D], drawn as the module docstring says."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    out = []
    for i in range(4):
        x = torch.randn((B, N, H, D), generator=gen, dtype=torch.float32)
        if i < 2 and qk_scale != 1.0:
            x.mul_(qk_scale)
        out.append(x.to(torch.bfloat16))
        del x
    return tuple(out)


def random_grad(B: int, N: int, H: int, D: int, seed: int):
    """Output gradient for the backward pass: bf16 CPU tensor [B, N, H, D],
    iid N(0, 1) from its own seeded generator (drawn after nothing else)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    x = torch.randn((B, N, H, D), generator=gen, dtype=torch.float32)
    return x.to(torch.bfloat16)


def random_projection(B: int, N: int, C: int, H: int, D: int, seed: int):
    """(x, w): hidden states x [B, N, C] iid N(0, 1) and stacked weights
    w [4, H*D, C] iid N(0, 1/C) (so each projection is ~N(0, 1) like the
    mixer's own inputs), drawn in that order from one seeded CPU generator
    in fp32 and rounded to bf16."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    x = torch.randn((B, N, C), generator=gen, dtype=torch.float32).to(torch.bfloat16)
    w = torch.randn((4, H * D, C), generator=gen, dtype=torch.float32)
    w = w.mul_(C ** -0.5).to(torch.bfloat16)
    return x, w


def make_projection(w: Workload, seed: int | None = None):
    """Seeded (x, w) of a projection workload."""
    return random_projection(w.B, w.N, w.C, w.H, w.D, w.seed if seed is None else seed)


def make_inputs(w: Workload, seed: int | None = None):
    """Seeded inputs of a named workload (seed defaults to the workload's own)."""
    return random_inputs(w.B, w.N, w.H, w.D, w.seed if seed is None else seed, w.qk_scale)
