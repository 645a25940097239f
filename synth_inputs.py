"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds no arithmetic of the quantization method: it draws numbers
from numpy's default_rng (PCG64) and rounds them to bf16 with torch's
round-to-nearest-even conversion, returning uint16 bit patterns.  Both the
oracle and the HIP library receive exactly these bits.

Workload shapes (the decode and prefill projections of a hidden-5120 model
with intermediate size 25600, and an MXFP4 model with hidden 2880):

  affine_small   x[1,512] ~ N(0,1), W[1024,512] ~ N(0,0.02^2), seed 1
  nvfp4_act      X[4096,5120] ~ N(0,1) with exactly floor(1% * numel)
                 positions (drawn without replacement) set to +-20, seed 2
  affine_decode  x[1,5120] ~ N(0,1), W_up[25600,5120] and W_down[5120,25600]
                 ~ N(0,0.02^2), seed 3
  mxfp4          W[5760,2880] ~ N(0,0.02^2), x[M,2880] ~ N(0,1), seed 4
  nvfp4_prefill  X[M,5120], W[25600,5120] ~ N(0,0.02^2), seed 5
"""
from __future__ import annotations

import numpy as np
import torch


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even, torch) -> uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return to_bf16_bits(a)


def rng_for(seed: int, stream: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


# ---------------------------------------------------------------- workloads

def affine_small():
    rng = rng_for(1)
    x = normal_bf16(rng, (1, 512))
    w = normal_bf16(rng, (1024, 512), 0.02)
    return x, w


def nvfp4_activations(rows: int = 4096, cols: int = 5120, seed: int = 2,
                      frac: float = 0.01, outlier: float = 20.0):
    rng = rng_for(seed)
    a = rng.standard_normal(size=(rows, cols), dtype=np.float32)
    n = rows * cols
    k = int(np.floor(frac * n))
    if k:
        pos = rng.choice(n, size=k, replace=False)
        sign = np.where(rng.random(k) < 0.5, -1.0, 1.0).astype(np.float32)
        a.reshape(-1)[pos] = sign * np.float32(outlier)
    return to_bf16_bits(a)


def affine_decode(which: str = "up", seed: int = 3):
    """x[1,K] and one weight matrix: 'up' [25600,5120] or 'down' [5120,25600]."""
    shapes = {"up": (25600, 5120), "gate": (25600, 5120), "down": (5120, 25600)}
    N, K = shapes[which]
    stream = {"up": 1, "gate": 2, "down": 3}[which]
    x = normal_bf16(rng_for(seed, 0), (1, K))
    w = normal_bf16(rng_for(seed, stream), (N, K), 0.02)
    return x, w


def mxfp4_weights(N: int = 5760, K: int = 2880, seed: int = 4):
    return normal_bf16(rng_for(seed, 1), (N, K), 0.02)


def mxfp4_activations(M: int, K: int = 2880, seed: int = 4):
    return normal_bf16(rng_for(seed, 100 + M), (M, K))


def nvfp4_prefill(M: int = 2048, N: int = 25600, K: int = 5120, seed: int = 5):
    x = normal_bf16(rng_for(seed, 100 + M), (M, K), 0.02)
    w = normal_bf16(rng_for(seed, 1), (N, K), 0.02)
    return x, w


def generic(shape, std: float = 1.0, seed: int = 0, stream: int = 0):
    """Any shape, for parity cases at oracle-friendly sizes."""
    return normal_bf16(rng_for(seed, stream), shape, std)


def random_words(shape, seed: int = 0, stream: int = 0) -> np.ndarray:
    """Uniform random uint32 words: the random input of stochastic-rounding
    quantize (one word per element), passed to both the kernel and the
    oracle."""
    return rng_for(seed, 1000 + stream).integers(0, 1 << 32, size=shape, dtype=np.uint32)


def torch_normal_bf16(shape, std: float, seed: int, device) -> torch.Tensor:
    """Device-side draw (torch's Philox generator) for large benchmark sweeps
    whose numbers never meet the oracle; returns a bf16 tensor on `device`."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return (t * std).to(torch.bfloat16)
