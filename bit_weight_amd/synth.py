"""Seeded synthetic inputs for the Sherry ternary matmul.

This module only draws random numbers; it holds none of the method's
arithmetic (no quantization, packing, lookup or product).  Both the GPU path
and the CPU oracle consume exactly the tensors it returns.

Workloads are LLaMA-shaped layers (no dataset or trained weights are used):

  name  M    K      N      weights                          activations
  1     1    256    256    Normal(0, 0.02)                  Normal(0, 1)
  2a    1    4096   4096   Normal(0, 0.02)                  Normal(0, 1)
  2b    4    4096   4096   same W as 2a                     Normal(0, 1)
  2c    16   4096   4096   same W as 2a                     Normal(0, 1)
  3a    1    4096   11008  Normal(0, 0.1), 1% -> +-5.0      Normal(0, 1)
  3b    1    11008  4096   Normal(0, 0.1), 1% -> +-5.0      Normal(0, 1)
  4     8    8192   28672  Normal(0, 0.02)                  Normal(0, 1)
  5     512  4096   14336  Normal(0, 0.02)                  Normal(0, 1), 20
                                                            channels x20

The spike distribution (Normal(0,0.1) with 1% of entries replaced by +-5.0)
is the synthetic long-tailed weight model of the ChenRT page (gitcode.csdn.net,
§3.1 experimental setup).  Every entry is replaced independently with
probability 0.01; the spike's sign is + or - with equal probability.  For
workload 5, round(0.005*K) channel indices are drawn without replacement and
multiplied by 20 for every token.
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    w_std: float
    w_spikes: bool
    x_outlier_channels: bool
    seed_w: int
    seed_x: int

    @property
    def packed_bytes(self) -> int:
        return self.N * self.K * 5 // 32

    @property
    def description(self) -> str:
        return (f"{self.name}: M={self.M}, K={self.K}, N={self.N}, "
                f"W~N(0,{self.w_std})" + (" +1% +-5.0 spikes" if self.w_spikes else "")
                + (", x outlier channels x20" if self.x_outlier_channels else ""))


WORKLOADS = {
    "1": Workload("1", 1, 256, 256, 0.02, False, False, 1001, 2001),
    "2a": Workload("2a", 1, 4096, 4096, 0.02, False, False, 1002, 2002),
    "2b": Workload("2b", 4, 4096, 4096, 0.02, False, False, 1002, 2003),
    "2c": Workload("2c", 16, 4096, 4096, 0.02, False, False, 1002, 2004),
    "3a": Workload("3a", 1, 4096, 11008, 0.1, True, False, 1005, 2005),
    "3b": Workload("3b", 1, 11008, 4096, 0.1, True, False, 1006, 2006),
    "4": Workload("4", 8, 8192, 28672, 0.02, False, False, 1007, 2007),
    "5": Workload("5", 512, 4096, 14336, 0.02, False, True, 1008, 2008),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def weights(N: int, K: int, std: float, spikes: bool, seed: int) -> torch.Tensor:
    """fp32 [N,K] on the CPU: Normal(0, std), optionally 1% +-5.0 spikes."""
    g = _gen(seed)
    W = torch.randn((N, K), generator=g, dtype=torch.float32) * std
    if spikes:
        hit = torch.rand((N, K), generator=g) < 0.01
        sign = torch.where(torch.rand((N, K), generator=g) < 0.5, -1.0, 1.0)
        W = torch.where(hit, 5.0 * sign, W)
    return W.contiguous()


def activations(M: int, K: int, seed: int, outlier_channels: bool = False) -> torch.Tensor:
    """fp32 [M,K] on the CPU: Normal(0,1), optionally round(0.005K) channels x20."""
    g = _gen(seed)
    x = torch.randn((M, K), generator=g, dtype=torch.float32)
    if outlier_channels:
        n_out = int(round(0.005 * K))
        ch = torch.randperm(K, generator=g)[:n_out]
        x[:, ch] *= 20.0
    return x.contiguous()


def int8_uniform(M: int, K: int, seed: int, lo: int = -128, hi: int = 127) -> torch.Tensor:
    """int8 [M,K] uniform on [lo, hi] (edge-case activations, includes -128)."""
    g = _gen(seed)
    return torch.randint(lo, hi + 1, (M, K), generator=g, dtype=torch.int16).to(torch.int8)


def workload_weights(w: Workload) -> torch.Tensor:
    return weights(w.N, w.K, w.w_std, w.w_spikes, w.seed_w)


def workload_activations(w: Workload) -> torch.Tensor:
    return activations(w.M, w.K, w.seed_x, w.x_outlier_channels)


def sha256(t: torch.Tensor) -> str:
    return hashlib.sha256(t.contiguous().numpy().tobytes()).hexdigest()
