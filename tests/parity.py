"""Shared helpers of the GPU parity tests: tolerances and host<->device moves.

Tolerances (the oracle is exact fp64; the GPU accumulates in fp32):
  * fp32 outputs:  max_i |g_i - o_i| / max(|o_i|, d_i) <= 2e-3, where d_i is the
    |.|-magnitude of the sum that produced o_i (the componentwise error scale
    of a dot product; for GELU outputs multiplied by GELU's Lipschitz bound
    1.13).
  * bf16 outputs:  |g - o| <= ulp_bf16(o) + 1e-2 and, so that tiny outputs are
    not waved through, |g - o| <= ulp_bf16(o) + 2e-3 max(|o|, d).
  * fp8 codes and scales of the cast: bit-identical.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads as W

REL_TOL = 2e-3
BF16_ABS = 1e-2
GELU_LIP = 1.13


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to("cuda")


def bf16_dev(bits):
    return dev(np.ascontiguousarray(bits, np.uint16)).view(torch.bfloat16)


def host(t):
    return t.detach().to("cpu").contiguous()


def bf16_host_f64(t):
    return W.bf16_bits_to_f32(host(t).view(torch.int16).numpy().view(np.uint16)).astype(np.float64)


def ulp_bf16(v):
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** -133)))
    return np.exp2(np.maximum(e, -133) - 7)


def check_f32(got, want, mag, what=""):
    got = np.asarray(got, np.float64)
    err = np.abs(got - want)
    scale = np.maximum(np.abs(want), mag)
    rel = err / np.where(scale > 0, scale, np.inf)
    worst = float(rel.max()) if rel.size else 0.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert worst <= REL_TOL, f"{what}: max rel err {worst:.3e} > {REL_TOL} at {np.unravel_index(rel.argmax(), rel.shape)}"
    return worst


def check_bf16(got, want, mag, what=""):
    got = np.asarray(got, np.float64)
    err = np.abs(got - want)
    u = ulp_bf16(want)
    lit = err <= u + BF16_ABS
    scaled = err <= u + REL_TOL * np.maximum(np.abs(want), mag)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    bad = ~(lit & scaled)
    assert not bad.any(), (f"{what}: {int(bad.sum())} bf16 outputs out of tolerance; first at "
                           f"{np.argwhere(bad)[0]} got {got[bad][0]} want {want[bad][0]}")


def scale_ld(rows):
    """Leading dimension of block-major scales, as the library reports it."""
    import fp8_linear_layer_amd as te
    return te.scale_ld(rows)


def sdev(s, fill=0.0):
    """Row-major oracle scales [rows][K/128] -> block-major device array [K/128][scale_ld(rows)].

    The padding rows carry `fill`, so a kernel that read them would show it.
    """
    s = np.asarray(s, np.float32)
    rows, nkb = s.shape
    bm = np.full((nkb, scale_ld(rows)), fill, np.float32)
    bm[:, :rows] = s.T
    return dev(bm)


def shost(t, rows):
    """Block-major device scales -> row-major numpy [rows][K/128] (the padding is dropped)."""
    return t.cpu().numpy()[:, :rows].T.copy()


def cast_host(bits, fmt, pow2=False):
    """Oracle cast on the host -> (q, s) numpy."""
    return oracle.cast_per_token(bits, fmt, pow2)


def to_dev_operand(q, s):
    return dev(q), sdev(s)
