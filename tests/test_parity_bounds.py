"""The fp32 tolerance of the GPU parity tests can tell fp32 accumulation from a reduced-precision
one (CPU only).

The products of a K = 4096 GEMM on N(0, 1) operands cast to e4m3 are accumulated here the way the
kernels do it (a 128-term sum per block, then one promotion per block), once in fp32 and once with
the running sum rounded to bf16 after every block.  The block sum is given the matrix core's
measured imprecision on top (each block's sum off by 2^-15.6 of its |.|-magnitude, the largest error
the GPU suite shows).  The floored relative rule alone passes both; the accumulation bound that
check_f32 adds passes the fp32 emulation and rejects the bf16 one, a dropped block, and a promotion
that forgets one of the two scales.  The quantised-store check rejects a code one step off.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import E_MMA, U32, chain_gemm, check_f32, check_quant, f32_stats, REL_TOL

K = 4096


def _operands(M=40, N=36):
    s = np.random.SeedSequence(777).spawn(2)
    qa, sa = oracle.cast_per_token(W.normal_bf16(s[0], (M, K)), oracle.E4M3)
    qb, sb = oracle.cast_per_token(W.normal_bf16(s[1], (N, K)), oracle.E4M3)
    return qa, sa, qb, sb


def _tree32(p):
    """Sum over the last axis (length 128) as a binary tree in fp32."""
    p = p.astype(np.float32)
    while p.shape[-1] > 1:
        p = (p[..., 0::2] + p[..., 1::2]).astype(np.float32)
    return p[..., 0]


def _emulate(qa, sa, qb, sb, mode):
    A, B = oracle.decode(qa, oracle.E4M3), oracle.decode(qb, oracle.E4M3)
    M, N = A.shape[0], B.shape[0]
    acc = np.zeros((M, N), np.float32)
    for kb in range(K // 128):
        blk = slice(128 * kb, 128 * (kb + 1))
        prod = A[:, None, blk] * B[None, :, blk]
        P = _tree32(prod)                                                   # exact products, fp32 tree
        # the matrix core's measured block-sum error, with the sign that hurts most
        P = (P + np.sign(P) * 2.0 ** -15.6 * np.abs(prod).sum(-1)).astype(np.float32)
        s = (sa[:, kb][:, None] * sb[:, kb][None, :]).astype(np.float32)    # sA sB in fp32
        if mode == "drop" and kb == 17:
            continue
        if mode == "one_scale":
            s = np.broadcast_to(sa[:, kb][:, None], (M, N)).astype(np.float32)
        t = (P * s).astype(np.float32)
        acc = (acc + t).astype(np.float32)
        if mode == "bf16":
            acc = W.bf16_bits_to_f32(W.f32_to_bf16_bits(acc)).astype(np.float32)
    return acc.astype(np.float64)


@pytest.fixture(scope="module")
def case():
    qa, sa, qb, sb = _operands()
    o, d = oracle.gemm_nt(qa, sa, oracle.E4M3, qb, sb, oracle.E4M3)
    return qa, sa, qb, sb, o, d


def test_fp32_accumulation_passes(case):
    qa, sa, qb, sb, o, d = case
    g = _emulate(qa, sa, qb, sb, "fp32")
    check_f32(g, o, d, "emulated fp32 promotion", chain_gemm(K))
    st = f32_stats(g, o, d)
    assert st["normwise"] < 1e-3


def test_bf16_accumulation_passes_the_floored_rule_but_not_the_bound(case):
    qa, sa, qb, sb, o, d = case
    g = _emulate(qa, sa, qb, sb, "bf16")
    st = f32_stats(g, o, d)
    assert st["max_rel"] <= REL_TOL          # what the floored 2e-3 rule alone would accept
    assert st["normwise"] > 1e-3             # yet the error is that of bf16, ~2^-9 of the result
    with pytest.raises(AssertionError, match="accumulation bound"):
        check_f32(g, o, d, "emulated bf16 promotion", chain_gemm(K))


@pytest.mark.parametrize("mode", ["drop", "one_scale"])
def test_gross_mistakes_fail(case, mode):
    qa, sa, qb, sb, o, d = case
    g = _emulate(qa, sa, qb, sb, mode)
    with pytest.raises(AssertionError):
        check_f32(g, o, d, f"emulated {mode}", chain_gemm(K))


def test_bound_scale_is_the_stated_one():
    """One unit of error at the bound's edge passes, just past it fails."""
    want = np.array([1.0, -2.0, 0.5])
    mag = np.array([3.0, 2.0, 0.5])
    chain = 10
    edge = E_MMA * mag + 4.0 * (chain + 2) * U32 * np.maximum(np.abs(want), mag)
    check_f32(want + 0.999 * edge, want, mag, "edge", chain)
    with pytest.raises(AssertionError):
        check_f32(want + 1.001 * edge, want, mag, "past edge", chain)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_quant_check_accepts_the_cast_and_rejects_a_code_one_step_off(fmt):
    rng = np.random.default_rng(5)
    y = (rng.standard_normal((8, 256)) * 3.0).astype(np.float32)
    q, s = oracle.cast_per_token_f32(y, fmt)
    check_quant(q, s, fmt, y.astype(np.float64), np.abs(y), "cast", chain=0)
    # a code whose mantissa field is neither all zeros nor all ones, moved one step away from the
    # exact value: the dequantised value is then a whole fp8 step off (twice the allowed half step)
    mbits = 3 if fmt == oracle.E4M3 else 2
    mant = q & ((1 << mbits) - 1)
    r, c = [int(v) for v in np.argwhere((mant != 0) & (mant != (1 << mbits) - 1) & (np.abs(y) > 1.0))[0]]
    exact = y[r, c] / s[r, c // 128]
    up = abs(oracle.decode(q[r, c], fmt)[()]) >= abs(exact)
    bad = q.copy()
    bad[r, c] = q[r, c] + 1 if up else q[r, c] - 1
    with pytest.raises(AssertionError, match="off the oracle"):
        check_quant(bad, s, fmt, y.astype(np.float64), np.abs(y), "cast with one bad code", chain=0)
