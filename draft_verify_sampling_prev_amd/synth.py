"""Seeded synthetic inputs for the DSpark per-step token path.

This module is shared by the GPU path's tests/benchmark and by the oracle's
tests.  It holds none of the method's arithmetic: it only draws random
tensors with the shapes, dtypes and distributions of the workloads, on the
CPU, with ``torch.Generator``.

The pages measure on real models and live traffic (GSM8K, HumanEval,
MT-Bench, DeepSeek-V4 traffic); none of that is available, and these seeded
tensors stand in for it.  The one property carried over from the pages is the
decay of acceptance along the block: the llm-wiki.hwlabs.dev explainer's
suffix-decay example table gives per-position acceptance of about
85/78/68/54/38/24/14/7 %, used as the "dsv4" workload's profile.

Recipe (every workload):
  T[b, k, :]  ~ N(0, 2^2)  target logits, rows k = 1..gamma+1
  L[b, k, :]  = T[b, k, :] + N(0, sigma_k^2)  backbone draft logits, k = 1..gamma
  A, Bm       ~ N(0, 0.02^2)  Markov factors [V][r] and [r][V]
  x0[b]       ~ uniform on [0, V)  last committed token
  z[b, k]     ~ N(mu_k, 1)  confidence logits
  temps[k]    = STS temperature per position (fitted on a held-out batch for the load sweep)
Values are drawn in float32 and rounded to bfloat16 (round-to-nearest-even)
for bf16 workloads.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

PHILOX_SEED = 0x0123456789ABCDEF

# Per-position acceptance example (llm-wiki.hwlabs.dev explainer, suffix-decay table).
SUFFIX_DECAY = (0.85, 0.78, 0.68, 0.54, 0.38, 0.24, 0.14, 0.07)


def _logit(p: float) -> float:
    return math.log(p / (1.0 - p))


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    gamma: int
    V: int
    r: int
    dtype: str               # "bf16" or "f32"
    sigma: tuple             # draft noise std per position k = 1..gamma
    mu: tuple                # confidence-logit mean per position
    temps: tuple             # STS temperature per position
    budget: int
    data_seed: int
    philox_seed: int = PHILOX_SEED

    def describe(self) -> dict:
        return {
            "workload": self.name, "B": self.B, "gamma": self.gamma, "V": self.V, "r": self.r,
            "dtype": self.dtype, "budget": self.budget,
        }


def _lin(a: float, b: float, gamma: int):
    return tuple(a + b * k for k in range(1, gamma + 1))


def tiny(B: int = 4, gamma: int = 5, V: int = 1024, r: int = 16, budget: int = 12, seed: int = 1000,
         dtype: str = "f32") -> Workload:
    """Tiny reference case: fp32, B=4, gamma=5, V=1024, r=16, budget 12."""
    return Workload("tiny", B, gamma, V, r, dtype, _lin(0.0, 0.5, gamma), _lin(1.5, -0.6, gamma),
                    _lin(1.0, 0.1, gamma), budget, seed)


def qwen3_4b(B: int = 64, gamma: int = 5, V: int = 151936, r: int = 256, seed: int = 1001) -> Workload:
    """Qwen3-4B-shaped single step: B=64, gamma=5, V=151936, r=256, bf16, budget 0.8*B*gamma."""
    return Workload("qwen3-4b-shaped", B, gamma, V, r, "bf16", _lin(0.0, 0.5, gamma), _lin(1.5, -0.6, gamma),
                    _lin(1.0, 0.1, gamma), int(0.8 * B * gamma), seed)


# Draft-noise levels at which the expected conditional acceptance sum_j min(p_t, p_d) of each position equals
# the suffix-decay example's 0.85/0.78/0.68/0.54/0.38, found by bisection on the held-out batch (seed 9002) by
# tests/calibrate_workloads.py (record: tests/golden/workload_calibration.json).
DSV4_SIGMA = (0.3782, 0.5584, 0.825, 1.2255, 1.7635)

# Sequential-temperature-scaling temperatures of the load-sweep workload, fitted left to right on the survival
# labels of one oracle step of its held-out batch (seed 9004, every drafted token verified) by
# tests/calibrate_workloads.py; the default before the fit was 1 + 0.1k.
LOAD_SWEEP_STS = (1.4887, 3.4002, 17.7361, 20.0, 0.3418, 0.3367, 0.05, 0.05)


def dsv4(B: int = 256, gamma: int = 5, V: int = 129280, r: int = 256, seed: int = 1002) -> Workload:
    """DeepSeek-V4-serving-shaped high-concurrency step: B=256, gamma=5, V=129280, r=256, bf16,
    budget 0.6*B*gamma, acceptance decaying per the suffix-decay example."""
    sig = tuple(DSV4_SIGMA[k] if k < len(DSV4_SIGMA) else DSV4_SIGMA[-1] for k in range(gamma))
    mu = tuple(_logit(SUFFIX_DECAY[k]) for k in range(gamma))
    return Workload("dsv4-serving-shaped", B, gamma, V, r, "bf16", sig, mu, tuple(1.0 for _ in range(gamma)),
                    int(0.6 * B * gamma), seed)


def long_block(gamma: int, B: int = 128, V: int = 151936, r: int = 256, seed: int = 1003) -> Workload:
    """Long-block sweep point: B=128, gamma in {4,8,12,16}, sigma_k = 0.4k, unbounded budget."""
    return Workload(f"long-block-g{gamma}", B, gamma, V, r, "bf16", _lin(0.0, 0.4, gamma), _lin(1.5, -0.6, gamma),
                    _lin(1.0, 0.1, gamma), B * gamma, seed)


def load_sweep(budget: int, B: int = 1024, gamma: int = 8, V: int = 129280, r: int = 256, seed: int = 1004,
               temps: Optional[tuple] = None) -> Workload:
    """Load-sweep point: B=1024, gamma=8, budget in {B, 2B, 4B, B*gamma}; confidence logits offset by +1
    (miscalibrated), temperatures fitted by sequential temperature scaling on the held-out batch."""
    t = temps if temps is not None else (LOAD_SWEEP_STS if gamma == len(LOAD_SWEEP_STS) else _lin(1.0, 0.1, gamma))
    return Workload(f"load-sweep-{budget}", B, gamma, V, r, "bf16", _lin(0.0, 0.5, gamma), _lin(2.5, -0.6, gamma),
                    t, budget, seed)


@dataclasses.dataclass
class Inputs:
    wl: Workload
    T: torch.Tensor       # [B][gamma+1][V]
    L: torch.Tensor       # [B][gamma][V]
    A: torch.Tensor       # [V][r]
    Bm: torch.Tensor      # [r][V]
    x0: torch.Tensor      # [B] int32
    z: torch.Tensor       # [B][gamma] float32
    temps: torch.Tensor   # [gamma] float32

    def to(self, device) -> "Inputs":
        return Inputs(self.wl, *(t.to(device) for t in (self.T, self.L, self.A, self.Bm, self.x0, self.z,
                                                          self.temps)))


def make_inputs(wl: Workload, seed: Optional[int] = None) -> Inputs:
    """Draw one batch of inputs for workload ``wl`` on the CPU."""
    g = torch.Generator().manual_seed(wl.data_seed if seed is None else seed)
    B, gamma, V, r = wl.B, wl.gamma, wl.V, wl.r
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    T32 = torch.randn((B, gamma + 1, V), generator=g, dtype=torch.float32).mul_(2.0)
    L32 = torch.randn((B, gamma, V), generator=g, dtype=torch.float32)
    sig = torch.tensor(wl.sigma, dtype=torch.float32).view(1, gamma, 1)
    L32.mul_(sig).add_(T32[:, :gamma, :])
    A = torch.randn((V, r), generator=g, dtype=torch.float32).mul_(0.02)
    Bm = torch.randn((r, V), generator=g, dtype=torch.float32).mul_(0.02)
    x0 = torch.randint(0, V, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    mu = torch.tensor(wl.mu, dtype=torch.float32).view(1, gamma)
    z = torch.randn((B, gamma), generator=g, dtype=torch.float32).add_(mu)
    temps = torch.tensor(wl.temps, dtype=torch.float32)
    return Inputs(wl, T32.to(dt), L32.to(dt), A.to(dt), Bm.to(dt), x0, z, temps)
