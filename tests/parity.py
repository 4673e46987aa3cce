"""Shared helpers of the GPU parity tests: tolerances and host<->device moves.

Tolerances (the oracle is exact fp64; the GPU accumulates in fp32):
  * fp32 outputs, two rules that must both hold:
      - the stated relative error, max_i |g_i - o_i| / max(|o_i|, d_i) <= 2e-3,
        where d_i is the |.|-magnitude of the sum that produced o_i (for GELU
        outputs multiplied by GELU's Lipschitz bound 1.13);
      - the accumulation bound
            |g_i - o_i| <= E_MMA d_i + C (n_i + 2) u max(|o_i|, d_i),
        u = 2^-24, C = 4, n_i the length of the longest chain of fp32 roundings
        that produced g_i (one per 128-deep block promoted, the scale product
        and the epilogue, see chain_gemm & co. below), and E_MMA = 2^-14 the
        error of the matrix core's own 128-term fp8 sum relative to the sum of
        its |terms|.  That sum is not exact in fp32: over the whole GPU parity
        suite its error reaches 2^-15.6 of the block's |.|-magnitude (worst at
        K = 128, where one block is the whole product), so E_MMA holds it with a
        3x margin; summed over blocks it is at most E_MMA d_i.  Only this rule
        sees the difference between fp32 promotion and reduced-precision
        accumulation: a bf16-rounded block accumulator passes the first rule at
        K = 4096 but misses this one ~17-fold (tests/test_parity_bounds.py).
    Reported next to them: the unfloored max |g - o| / |o|, how many elements
    took the floor d_i > |o_i|, and the norm-wise ||g - o||_inf / ||o||_inf.
  * bf16 outputs:  |g - o| <= ulp_bf16(o) + 1e-2 and, so that tiny outputs are
    not waved through, |g - o| <= ulp_bf16(o) + 2e-3 max(|o|, d).
  * fp8 codes and scales of the cast: bit-identical.
  * quantised stores (codes q and scales s written by an epilogue): besides
    the bit-exact match with the cast of the kernel's own fp32 result, the
    dequantised value is held to the fp64 oracle:
    |dec(q) s - o| <= ulp_fp8(dec(q)) s / 2 + the accumulation bound above + 4 u |o|
    (the fp32 value the codes were cast from may sit on the other side of a
    rounding midpoint than the exact one, by at most the accumulation bound).
"""
from __future__ import annotations

import os

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


U32 = 2.0 ** -24       # unit roundoff of fp32
ACC_C = 4.0            # safety factor of the fp32-accumulation bound
E_MMA = 2.0 ** -14     # the matrix core's 128-term fp8 sum, relative to its |.|-magnitude
BIAS_CHAIN = 1         # the bias add
GELU_CHAIN = 16        # GELU or GELU' evaluated with exp2 / reciprocal approximations (a few ulp each,
                       # amplified by the exponent's argument)

# Worst figures of every check_f32 call of the session, printed by conftest's summary hook.
REPORT: dict = {}


def chain_gemm(K, extra=0):
    """fp32 roundings along one GEMM output: a promotion per 128-deep block, the scale product,
    and `extra` epilogue steps (bias, GELU, +=)."""
    return (int(K) + 127) // 128 + 1 + extra


def chain_colsum(K, rows, extra=0):
    """A bias gradient: the summed outputs' own chain, then the sum over `rows` rows (four rows per
    lane in order, a 16-lane tree, then one add per 64-row wave slice)."""
    return chain_gemm(K, extra) + 4 + 4 + (int(rows) + 63) // 64


def chain_rowsum(K):
    """Row sums of a dequantised operand: a 16-term tree per lane and 1024-column step, the steps
    in order, then a 64-lane tree."""
    return (int(K) + 1023) // 1024 + 4 + 1 + 6


def f32_stats(got, want, mag):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want)
    scale = np.maximum(np.abs(want), mag)
    rel = err / np.where(scale > 0, scale, np.inf)
    nz = np.abs(want) > 0
    unfl = err[nz] / np.abs(want[nz]) if nz.any() else np.zeros(0)
    top = float(np.abs(want).max()) if want.size else 0.0
    return {
        "max_rel": float(rel.max()) if rel.size else 0.0,
        "max_rel_unfloored": float(unfl.max()) if unfl.size else 0.0,
        "n_floored": int((mag > np.abs(want)).sum()),
        "n": int(want.size),
        "normwise": float(err.max() / top) if top > 0 else float(err.max() if err.size else 0.0),
        "err": err, "scale": scale,
    }


def acc_bound(want, mag, chain, mma=True):
    """The accumulation bound of the module docstring (mma=False for sums formed without the matrix
    cores, e.g. a bias gradient checked against the column sums of the kernel's own output)."""
    scale = np.maximum(np.abs(want), mag)
    return (E_MMA * mag if mma else 0.0) + ACC_C * (np.asarray(chain, np.float64) + 2.0) * U32 * scale


def check_f32(got, want, mag, what="", chain=None, mma=True):
    """Both fp32 rules (see the module docstring); `chain` is the rounding-chain length n_i
    (a scalar or an array broadcasting against the outputs)."""
    assert chain is not None, "check_f32 needs the rounding-chain length of the outputs"
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    mag = np.asarray(mag, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    st = f32_stats(got, want, mag)
    bound = acc_bound(want, mag, chain, mma)
    over = st["err"] / np.where(bound > 0, bound, np.inf)
    acc_ratio = float(over.max()) if over.size else 0.0
    rec = REPORT.setdefault(what, {"calls": 0, "max_rel": 0.0, "max_rel_unfloored": 0.0, "normwise": 0.0,
                                   "acc_bound_ratio": 0.0, "n_floored": 0, "n": 0})
    rec["calls"] += 1
    for k in ("max_rel", "max_rel_unfloored", "normwise"):
        rec[k] = max(rec[k], st[k])
    rec["acc_bound_ratio"] = max(rec["acc_bound_ratio"], acc_ratio)
    rec["max_err_over_scale_u"] = max(rec.get("max_err_over_scale_u", 0.0), st["max_rel"] / U32)
    rec["n_floored"] += st["n_floored"]
    rec["n"] += st["n"]
    assert st["max_rel"] <= REL_TOL, (f"{what}: max rel err {st['max_rel']:.3e} > {REL_TOL} at "
                                      f"{np.unravel_index(np.argmax(st['err'] / st['scale']), want.shape)}")
    if os.environ.get("PARITY_MEASURE"):
        return st["max_rel"]     # (measuring run: record the ratio to the bound without asserting it)
    assert acc_ratio <= 1.0, (f"{what}: error {acc_ratio:.2f}x the accumulation bound (max rel "
                              f"{st['max_rel']:.3e}, norm-wise {st['normwise']:.3e}) at "
                              f"{np.unravel_index(over.argmax(), over.shape)}")
    return st["max_rel"]


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


def ulp_fp8(v, fmt):
    """Spacing of the fp8 grid at |v| (OCP E4M3FN: 3 mantissa bits, normals from 2^-6;
    E5M2: 2 mantissa bits, normals from 2^-14)."""
    import oracle
    mbits, emin = (3, -6) if fmt == oracle.E4M3 else (2, -14)
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** emin)))
    return np.exp2(np.maximum(e, emin) - mbits)


def check_quant(q, s, fmt, want, mag, what="", chain=None):
    """Quantised store held to the fp64 oracle: |dec(q) s - o| <= ulp_fp8(dec(q)) s / 2 + the
    fp32-accumulation bound + 4 u |o| (the scale's and the multiplier's roundings).  q [rows][N]
    codes, s [rows][N/128] row-major scales."""
    import oracle
    assert chain is not None
    dec = oracle.decode(q, fmt)
    sr = np.repeat(np.asarray(s, np.float64), 128, axis=1)
    got = dec * sr
    want = np.asarray(want, np.float64)
    err = np.abs(got - want)
    bound = 0.5 * ulp_fp8(dec, fmt) * sr + acc_bound(want, mag, chain) + 4 * U32 * np.abs(want)
    ratio = err / bound
    assert np.all(np.isfinite(got)), f"{what}: non-finite dequantised value"
    w = np.unravel_index(ratio.argmax(), ratio.shape)
    assert ratio.max() <= 1.0, (f"{what}: dequantised value off the oracle by {ratio.max():.2f}x the bound at {w} "
                                f"(got {got[w]}, want {want[w]})")
    return float(ratio.max())
