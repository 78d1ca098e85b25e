"""Seeded synthetic inputs for the dual-weight GLU projection.

This module only draws random numbers; it holds none of the projection's
arithmetic, and it is the one module that both the device path's tests and
the oracle's tests use.  Every tensor is bf16 (torch.bfloat16), drawn as fp32
normals and rounded to bf16 by torch's cast (to nearest, ties to even).

The workloads stand in for the pages' Qwen3.5-4B decode measurement (trained
weights and prompts are not used): the shapes of a 4B-class decoder MLP and
its neighbours, hidden ~ N(0, 1), weights ~ N(0, 0.02^2) (std 0.02, the usual
initializer range), plus the variations each workload names below.

Seeding: weights of one set come from ``torch.Generator(device).manual_seed(seed)``
drawing Wg then Wu; hidden rows come from a separate generator seeded
``seed + HIDDEN_SEED_OFFSET`` so they never share a stream with a weight set.
Draws on 'cpu' and on a GPU generator differ; a test that compares against the
oracle copies whatever it drew to the host first.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional, Tuple

import torch

HIDDEN_SEED_OFFSET = 1 << 40
GRAD_SEED_OFFSET = 2 << 40  # upstream gradients draw from their own stream
WEIGHT_STD = 0.02
OUTLIER_STD = 0.2
OUTLIER_FRAC = 0.01


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def hidden(M: int, K: int, seed: int, device="cpu", row0_scale: float = 1.0,
           std: float = 1.0) -> torch.Tensor:
    """Hidden rows [M, K] ~ N(0, std^2); row 0 multiplied by ``row0_scale`` (exact for powers of two)."""
    g = _gen(device, seed + HIDDEN_SEED_OFFSET)
    h = torch.randn((M, K), generator=g, device=device, dtype=torch.float32) * std
    if row0_scale != 1.0 and M > 0:
        h[0] *= row0_scale
    return h.to(torch.bfloat16)


def grad_out(M: int, N: int, seed: int, device="cpu", std: float = 1.0) -> torch.Tensor:
    """Upstream gradient rows [M, N] ~ N(0, std^2) for the backward (their own seed stream)."""
    g = _gen(device, seed + GRAD_SEED_OFFSET)
    return (torch.randn((M, N), generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)


def _one_weight(N: int, K: int, g: torch.Generator, device, std: float,
                outlier_frac: float, outlier_std: float) -> torch.Tensor:
    w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32) * std
    if outlier_frac > 0.0:
        mask = torch.rand((N, K), generator=g, device=device) < outlier_frac
        alt = torch.randn((N, K), generator=g, device=device, dtype=torch.float32) * outlier_std
        w = torch.where(mask, alt, w)
        del mask, alt
    return w.to(torch.bfloat16)


def weights(N: int, K: int, seed: int, device="cpu", std: float = WEIGHT_STD,
            outlier_frac: float = 0.0, outlier_std: float = OUTLIER_STD
            ) -> Tuple[torch.Tensor, torch.Tensor]:
    """(gate_w, up_w), each [N, K] in the nn.Linear layout.

    Entries ~ N(0, std^2); with ``outlier_frac`` > 0 each entry independently
    (Bernoulli mask) is redrawn from N(0, outlier_std^2) instead.
    """
    g = _gen(device, seed)
    wg = _one_weight(N, K, g, device, std, outlier_frac, outlier_std)
    wu = _one_weight(N, K, g, device, std, outlier_frac, outlier_std)
    return wg, wu


@dataclass(frozen=True)
class Workload:
    """One named workload: shapes, value recipe and the seeds its parity cases use."""
    name: str
    Ms: Tuple[int, ...]
    K: int
    N: int
    seeds: Tuple[int, ...]
    row0_scale: float = 1.0
    outlier_frac: float = 0.0
    layers: int = 1
    description: str = ""


WORKLOADS: Dict[str, Workload] = {
    "tail_k1024_n3000": Workload(
        "tail_k1024_n3000", (1,), 1024, 3000, (0,),
        description="M=1 K=1024 N=3000 (N not a multiple of 64)"),
    "decode_k2560_n9216": Workload(
        "decode_k2560_n9216", (1,), 2560, 9216, (0, 1, 2, 3, 4),
        description="M=1 K=2560 N=9216, a 4B-class decoder MLP gate/up (94.4 MB of weights)"),
    "stack32_k2560_n9216": Workload(
        "stack32_k2560_n9216", (1,), 2560, 9216, (0,), layers=32,
        description="32 distinct layers of K=2560 N=9216 called in layer order (3.02 GB)"),
    "batch_k4096_n12288": Workload(
        "batch_k4096_n12288", (2, 4, 8), 4096, 12288, (0, 1), row0_scale=8.0,
        description="M in {2,4,8} K=4096 N=12288, hidden row 0 scaled x8"),
    "mfma_k5120_n17408": Workload(
        "mfma_k5120_n17408", (16, 32), 5120, 17408, (0, 1), outlier_frac=OUTLIER_FRAC,
        description="M in {16,32} K=5120 N=17408, 1% of weights N(0,0.2^2) outliers"),
}


def case(workload: str, M: Optional[int] = None, seed: Optional[int] = None,
         device="cpu") -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """(hidden [M,K], gate_w [N,K], up_w [N,K]) of one single-layer workload case."""
    w = WORKLOADS[workload]
    M = w.Ms[0] if M is None else M
    seed = w.seeds[0] if seed is None else seed
    wg, wu = weights(w.N, w.K, seed, device=device, outlier_frac=w.outlier_frac)
    h = hidden(M, w.K, seed, device=device, row0_scale=w.row0_scale)
    return h, wg, wu


def stack_layer_seed(seed: int, layer: int) -> int:
    """Weight seed of layer ``layer`` in a decode stack drawn from ``seed``."""
    return seed * 1000 + layer


def stack_hidden(seed: int, layers: int, K: int, device="cpu") -> torch.Tensor:
    """Per-layer hidden vectors [layers, K]: one generator draws h_0 ... h_{L-1} in order."""
    return hidden(layers, K, seed, device=device)


def stack_weights(seed: int, layers: int, N: int, K: int, device="cpu"):
    """List of (gate_w, up_w) per layer of a decode stack."""
    return [weights(N, K, stack_layer_seed(seed, l), device=device) for l in range(layers)]
