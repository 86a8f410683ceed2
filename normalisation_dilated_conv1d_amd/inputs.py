"""Seeded synthetic inputs for the pre-norm dilated block and the Conv1d+GroupNorm sibling.

This module only draws random numbers. It holds none of the block's arithmetic, so
both the HIP path and the CPU oracle can be fed from it without sharing any of the
method. Everything is drawn in float32 on the CPU from a fixed ``torch.Generator``;
callers copy the tensors to the device themselves, so the GPU and the oracle see
identical bits.

Distributions (``N(0, s)`` means standard deviation ``s``, ``U(a, b)`` uniform):

pre-norm block, per sample count N, channels C, length L
    x ~ N(0, 1) (rounded to bfloat16, round-to-nearest-even, for the bf16 workload)
    running_mean ~ U(-0.5, 0.5), running_var ~ U(0.5, 1.5)
    gamma ~ U(0.5, 1.5), beta ~ N(0, 0.1), eps = 1e-5
    W[C, C, 3] ~ N(0, 1/sqrt(3C)), b[C] ~ N(0, 0.01)

Conv1d + GroupNorm, per N, C_in, C_out, T
    x ~ N(0, 1), W[C_out, C_in, 3] ~ N(0, 1/sqrt(3 C_in)), no bias
    gamma ~ U(0.5, 1.5), beta ~ N(0, 0.1), eps = 1e-5

Draw order is fixed (x, running_mean, running_var, gamma, beta, W, b for the block;
x, W, gamma, beta for the sibling), so a seed names one input set for good.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

EPS = 1e-5


@dataclass(frozen=True)
class Workload:
    """One benchmark configuration (shapes only)."""

    index: int
    kind: str  # "prenorm" or "groupnorm"
    name: str
    dims: dict = field(default_factory=dict)


# The five workloads the library is measured and checked on.
WORKLOADS = {
    0: Workload(0, "prenorm", "prenorm_tiny_N2_C16_L512_d128_f32",
                dict(N=2, C=16, L=512, d=128, dtype="f32")),
    1: Workload(1, "prenorm", "prenorm_N32_C256_L4096_d128_f32",
                dict(N=32, C=256, L=4096, d=128, dtype="f32")),
    2: Workload(2, "prenorm", "prenorm_dilation_sweep_N32_C256_L4096_f32",
                dict(N=32, C=256, L=4096, ds=(1, 8, 512, 2048), dtype="f32")),
    3: Workload(3, "groupnorm", "conv1d_groupnorm_N16_Cin128_Cout256_T1024_G32_f32",
                dict(N=16, C_in=128, C_out=256, T=1024, G=32, padding=1, dilation=1)),
    4: Workload(4, "prenorm", "prenorm_wide_N16_C512_L16384_d128_bf16",
                dict(N=16, C=512, L=16384, d=128, dtype="bf16")),
}


def seed_for(config: int, sub: int = 0) -> int:
    """Seed convention: 1000 * workload index + sub-index."""
    return 1000 * config + sub


def prenorm_inputs(N: int, C: int, L: int, seed: int, *, bf16: bool = False,
                   eps: float = EPS) -> dict:
    """Draw one input set for the pre-norm block. All tensors are float32 on the CPU,
    except ``x`` which is bfloat16 when ``bf16`` is set."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(N, C, L, generator=g, dtype=torch.float32)
    running_mean = torch.rand(C, generator=g) - 0.5
    running_var = torch.rand(C, generator=g) + 0.5
    gamma = torch.rand(C, generator=g) + 0.5
    beta = torch.randn(C, generator=g) * 0.1
    W = torch.randn(C, C, 3, generator=g) * (1.0 / math.sqrt(3 * C))
    b = torch.randn(C, generator=g) * 0.01
    if bf16:
        x = x.to(torch.bfloat16)
    return dict(x=x, running_mean=running_mean, running_var=running_var,
                gamma=gamma, beta=beta, eps=eps, W=W, b=b)


def groupnorm_inputs(N: int, C_in: int, C_out: int, T: int, seed: int, *,
                     with_bias: bool = False, eps: float = EPS) -> dict:
    """Draw one input set for Conv1d(k=3) + GroupNorm. float32 CPU tensors."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(N, C_in, T, generator=g, dtype=torch.float32)
    W = torch.randn(C_out, C_in, 3, generator=g) * (1.0 / math.sqrt(3 * C_in))
    gamma = torch.rand(C_out, generator=g) + 0.5
    beta = torch.randn(C_out, generator=g) * 0.1
    bias = (torch.randn(C_out, generator=g) * 0.01) if with_bias else None
    return dict(x=x, W=W, bias=bias, gamma=gamma, beta=beta, eps=eps)
