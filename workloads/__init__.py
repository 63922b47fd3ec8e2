"""Seeded synthetic inputs for the QLoRA NF4 linear layer.

This module holds the workload definitions and the random-input generators
shared by the tests, the benchmark and the smoke entry point.  It contains none
of the method's arithmetic: it draws normal variates and hands them over as
data (fp32 weights, bf16 bit patterns for the activations and adapters).  The
bf16 rounding of inputs uses torch's CPU conversion so that neither the oracle
nor the HIP library supplies it.

Workloads (shapes and distributions of the layer the pages describe; no public
dataset or benchmark is involved):
  single     W0 256x512, M=16, r=8, alpha=16
  layer4096  W0 4096x4096 (the pages' 4096x4096 example layer), M=4096
             (batch 4 x sequence 1024), r=8, alpha=16
  decode     W0 4096x4096 and 14336x4096, M in {1, 4, 16}, r=16, alpha=32,
             forward only
  llama7b    q,k,v,o 4096x4096; gate, up 11008x4096; down 4096x11008;
             M=2048, r=64, alpha=16
  llama65b   q,k,v,o 8192x8192; gate, up 22016x8192; down 8192x22016;
             M=4096, r=64, alpha=16

Distributions: W0 ~ N(0, 0.02^2) fp32; A ~ N(0, 1/r); B ~ N(0, 0.01^2) (nonzero
so that the adapter path is exercised); x, dY ~ N(0, 1).  Each projection draws
from numpy's PCG64 seeded with SeedSequence([workload_seed, projection_index]),
in the order W0, A, B, x, dY, as float32 normals scaled in fp32; x, A, B and dY
are then rounded once to bf16.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Projection:
    name: str
    d: int          # output features (rows of W0)
    k: int          # input features (columns of W0)


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    projections: tuple
    m: tuple        # token counts (several only for the decode workload)
    r: int
    alpha: float
    backward: bool = True
    note: str = field(default="", compare=False)


WORKLOADS = {
    "single": Workload("single", 0, (Projection("proj", 256, 512),), (16,), 8, 16.0),
    "layer4096": Workload("layer4096", 1, (Projection("proj", 4096, 4096),), (4096,), 8, 16.0),
    "decode": Workload("decode", 2, (Projection("4096x4096", 4096, 4096),
                                     Projection("14336x4096", 14336, 4096)),
                       (1, 4, 16), 16, 32.0, backward=False),
    "llama7b": Workload("llama7b", 3, (
        Projection("q", 4096, 4096), Projection("k", 4096, 4096), Projection("v", 4096, 4096),
        Projection("o", 4096, 4096), Projection("gate", 11008, 4096),
        Projection("up", 11008, 4096), Projection("down", 4096, 11008)), (2048,), 64, 16.0),
    "llama65b": Workload("llama65b", 4, (
        Projection("q", 8192, 8192), Projection("k", 8192, 8192), Projection("v", 8192, 8192),
        Projection("o", 8192, 8192), Projection("gate", 22016, 8192),
        Projection("up", 22016, 8192), Projection("down", 8192, 22016)), (4096,), 64, 16.0),
}

W0_STD = 0.02
B_STD = 0.01


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (torch CPU conversion, nearest-even); uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_as_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (for feeding float64 references)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class LayerInputs:
    w0: np.ndarray          # float32 [d, k]
    a: np.ndarray           # uint16 bf16 bits [r, k]
    b: np.ndarray           # uint16 bf16 bits [d, r]
    x: np.ndarray           # uint16 bf16 bits [m, k]
    dy: np.ndarray | None   # uint16 bf16 bits [m, d]


def make_layer(seed: int, proj_index: int, d: int, k: int, m: int, r: int,
               with_dy: bool = True, w0_std: float = W0_STD, b_std: float = B_STD) -> LayerInputs:
    """Draw one projection's inputs (order W0, A, B, x, dY)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, proj_index]))
    w0 = rng.standard_normal((d, k), dtype=np.float32)
    w0 *= np.float32(w0_std)
    a = rng.standard_normal((r, k), dtype=np.float32) * np.float32(1.0 / np.sqrt(r))
    b = rng.standard_normal((d, r), dtype=np.float32) * np.float32(b_std)
    x = rng.standard_normal((m, k), dtype=np.float32)
    dy = rng.standard_normal((m, d), dtype=np.float32) if with_dy else None
    return LayerInputs(w0=w0, a=to_bf16_bits(a), b=to_bf16_bits(b), x=to_bf16_bits(x),
                       dy=None if dy is None else to_bf16_bits(dy))


def workload_layer(name: str, proj_index: int = 0, m: int | None = None) -> LayerInputs:
    """Inputs of one projection of a named workload (decode draws x with M=16;
    smaller M use its leading rows)."""
    wl = WORKLOADS[name]
    p = wl.projections[proj_index]
    mm = max(wl.m) if m is None else m
    return make_layer(wl.seed, proj_index, p.d, p.k, mm, wl.r, with_dy=wl.backward)


def random_weights(seed: int, shape, std: float = W0_STD) -> np.ndarray:
    """Plain N(0, std^2) fp32 weights for shape sweeps and edge cases."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x5EED]))
    out = rng.standard_normal(shape, dtype=np.float32)
    out *= np.float32(std)
    return out


def device_normal(seed: int, shape, std: float = W0_STD, device: str = "cuda"):
    """N(0, std^2) fp32 drawn on the device by torch's seeded generator, for
    inputs too large to draw on the host in a test's time (2^30 weights)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).mul_(std)


def random_bf16(seed: int, shape, std: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0xBF16]))
    return to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))
