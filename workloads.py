"""Seeded synthetic inputs for the scaled-FP8 Linear GEMMs.

This module only draws random numbers and rounds them to bf16 storage; it holds
none of the method's arithmetic (no casting to fp8, no GEMM, no epilogue).  Both
the oracle side (tests, CPU baseline) and the GPU side (tests, benchmark) take
their inputs from here.

Shapes and value distributions follow the five workloads of the fp8 Linear
layer in training (dense fprop, dgrad and wgrad at transformer sizes, and the
K-grouped MoE wgrad); the distributions the descriptions leave open are fixed
here and listed in the design notes.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(seed: np.random.SeedSequence, shape, std: float = 1.0) -> np.ndarray:
    """bf16 bits of N(0, std^2) draws (drawn in fp32, rounded to bf16)."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def uniform_bf16(seed: np.random.SeedSequence, shape) -> np.ndarray:
    """bf16 bits of U[0, 1) draws."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.random(shape, dtype=np.float32))


def normal_f32(seed: np.random.SeedSequence, shape, std: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def moe_group_k(seed, experts: int = 8, total: int = 32768, block: int = 128) -> np.ndarray:
    """Per-expert token counts: multinomial over experts in blocks of `block`, summing to `total`."""
    rng = np.random.default_rng(seed)
    counts = rng.multinomial(total // block, [1.0 / experts] * experts)
    return counts.astype(np.int64) * block


def spawn(seed: int, n: int):
    return np.random.SeedSequence(seed).spawn(n)


@dataclass
class Workload:
    name: str
    seed: int
    shapes: dict = field(default_factory=dict)


# The five workloads (rows x cols; every operand is contraction-contiguous).
TINY_FPROP = Workload("tiny-fprop-256x256x512", 1,
                      dict(M=256, N=256, K=512, x_std=1.0, w_std=1.0, b_std=0.1))
DENSE_WGRAD = Workload("dense-wgrad-7168x2112x4096", 2,
                       dict(M=7168, N=2112, K=4096, a_std=1.0, b_std=1.0))
FPROP = Workload("fprop-8192x14336x4096", 3,
                 dict(M=8192, N=14336, K=4096, x_std=1.0, w_std=0.02, b_std=0.1))
DGRAD = Workload("dgrad-8192x4096x14336", 4,
                 dict(M=8192, N=4096, K=14336, dy_std=1e-3, w_std=0.02, z_std=1.28))
KGROUPED = Workload("kgrouped-wgrad-8x2048x7168-sumK32768", 5,
                    dict(G=8, M=2048, N=7168, sumK=32768, a_std=1.0, b_std=1.0))


def tiny_fprop_inputs():
    s = spawn(TINY_FPROP.seed, 4)
    sh = TINY_FPROP.shapes
    return dict(x=normal_bf16(s[0], (sh["M"], sh["K"])),
                w=normal_bf16(s[1], (sh["N"], sh["K"])),
                b=normal_bf16(s[2], (sh["N"],), sh["b_std"]),
                out0=normal_f32(s[3], (sh["M"], sh["N"])))


def dense_wgrad_inputs(M=None, N=None, K=None):
    sh = DENSE_WGRAD.shapes
    M = M or sh["M"]; N = N or sh["N"]; K = K or sh["K"]
    s = spawn(DENSE_WGRAD.seed, 3)
    return dict(a=normal_bf16(s[0], (M, K)), b=normal_bf16(s[1], (N, K)),
                out0=normal_f32(s[2], (M, N)))


def fprop_inputs(M=None, N=None, K=None):
    sh = FPROP.shapes
    M = M or sh["M"]; N = N or sh["N"]; K = K or sh["K"]
    s = spawn(FPROP.seed, 3)
    return dict(x=normal_bf16(s[0], (M, K), sh["x_std"]),
                w=normal_bf16(s[1], (N, K), sh["w_std"]),
                b=normal_bf16(s[2], (N,), sh["b_std"]))


def dgrad_inputs(M=None, N=None, K=None):
    """dX GEMM operands (dY [M,K] e5m2 source, W^T [N,K]) plus the dGELU/bias-grad
    case at the pre-activation shape: dO [M, N2] (N2 = N), W2^T [K, N2] and Z [M, K]."""
    sh = DGRAD.shapes
    M = M or sh["M"]; N = N or sh["N"]; K = K or sh["K"]
    s = spawn(DGRAD.seed, 5)
    return dict(dy=normal_bf16(s[0], (M, K), sh["dy_std"]),
                wt=normal_bf16(s[1], (N, K), sh["w_std"]),
                do=normal_bf16(s[2], (M, N), sh["dy_std"]),
                w2t=normal_bf16(s[3], (K, N), sh["w_std"]),
                z=normal_bf16(s[4], (M, K), sh["z_std"]))


def kgrouped_inputs(G=None, M=None, N=None, sumK=None):
    sh = KGROUPED.shapes
    G = G or sh["G"]; M = M or sh["M"]; N = N or sh["N"]; sumK = sumK or sh["sumK"]
    s = spawn(KGROUPED.seed, 4)
    return dict(a=normal_bf16(s[0], (M, sumK), sh["a_std"]),
                b=normal_bf16(s[1], (N, sumK), sh["b_std"]),
                group_k=moe_group_k(s[2], G, sumK),
                out0=normal_f32(s[3], (G, M, N)))
