"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test ties the oracle to something other than its own formulas: values the
pages print, hand-derived fixtures, library routines (torch's float8 casts,
numpy matmul, torch's tanh-GELU and autograd), closed forms and brute force.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")
FMTS = {oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}


def torch_decode(codes, fmt):
    """Library decode of fp8 codes (torch's float8 dtypes), independent of the oracle."""
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(FMTS[fmt])
    return t.to(torch.float64).numpy()


def dequant(q, s, fmt):
    """Library dequantisation: decode with torch, multiply each 128-column group by its scale."""
    return torch_decode(q, fmt) * np.repeat(s.astype(np.float64), 128, axis=1)


def bits(x):
    return W.f32_to_bf16_bits(np.asarray(x, np.float32))


# ------------------------------------------------------------------ codecs
@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_decode_all_codes_match_torch(fmt):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode(codes, fmt)
    ref = torch_decode(codes, fmt)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_decode_worked_values():
    names = {"e4m3": oracle.E4M3, "e5m2": oracle.E5M2}
    n = 0
    with open(os.path.join(GOLD, "fp8_worked_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if not line:
                continue
            fmt, code, val = names[line[0]], int(line[1], 16), line[2]
            got = oracle.decode([code], fmt)[0]
            if val == "nan":
                assert np.isnan(got)
            else:
                want = float(val)
                assert got == want and np.signbit(got) == np.signbit(want), (line, got)
            n += 1
    assert n >= 20
    assert oracle.fp8_max(oracle.E4M3) == 448.0 and oracle.fp8_max(oracle.E5M2) == 57344.0


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_encode_matches_torch_in_range(fmt):
    """Round-to-nearest-even against torch's float8 cast for in-range fp32 values.

    Covers every code's exact value, every midpoint between neighbours and one
    fp32 ulp either side of it, and a million random bit patterns."""
    fmax = oracle.fp8_max(fmt)
    vals = torch_decode(np.arange(256, dtype=np.uint8), fmt)
    pos = np.sort(vals[np.isfinite(vals) & (vals >= 0)])
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    cand = [pos.astype(np.float32), mids, np.nextafter(mids, np.float32(0)),
            np.nextafter(mids, np.float32(np.inf))]
    rng = np.random.default_rng(7)
    rb = rng.integers(0, 2**32, size=1_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    cand.append(rb[np.isfinite(rb)])
    v = np.concatenate([np.concatenate(cand), -np.concatenate(cand)]).astype(np.float32)
    v = v[np.abs(v) <= fmax]
    ours = oracle.encode(v, fmt)
    ref = torch.from_numpy(v).to(FMTS[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref), np.flatnonzero(ours != ref)[:10]


@pytest.mark.parametrize("fmt,maxcode", [(oracle.E4M3, 0x7E), (oracle.E5M2, 0x7B)])
def test_encode_saturates_and_keeps_sign(fmt, maxcode):
    fmax = oracle.fp8_max(fmt)
    big = np.array([fmax * 1.03, fmax * 2, 3e38, np.inf], np.float32)
    assert (oracle.encode(big, fmt) == maxcode).all()
    assert (oracle.encode(-big, fmt) == (0x80 | maxcode)).all()
    assert oracle.encode(np.array([-0.0, -1e-30], np.float32), fmt).tolist() == [0x80, 0x80]
    # round trip of every finite code
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.decode(codes, fmt)
    fin = np.isfinite(vals)
    assert np.array_equal(oracle.encode(vals[fin].astype(np.float32), fmt), codes[fin])


# ------------------------------------------------------------------ cast
def test_cast_hand_derived_group():
    x = np.zeros(128, np.float32)
    want = np.zeros(128, np.uint8)
    with open(os.path.join(GOLD, "cast_e4m3_amax448_group.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if not line:
                continue
            i, v, c = int(line[0]), float(line[1]), int(line[2], 16)
            x[i] = v
            want[i] = c
    xb = bits(x)
    assert np.array_equal(W.bf16_bits_to_f32(xb), x)  # every listed value is exact in bf16
    q, s = oracle.cast_per_token(xb[None, :], oracle.E4M3)
    assert s[0, 0] == np.float32(1.0)
    assert np.array_equal(q[0], want), np.flatnonzero(q[0] != want)


def test_cast_ones_example_codes_and_scale():
    """The ones operand of the pages' wgrad example: every code is the e4m3 maximum."""
    q, s = oracle.cast_per_token(bits(np.ones((4, 512))), oracle.E4M3)
    assert (q == 0x7E).all()
    assert (s.view(np.uint32) == 0x3B124925).all()  # fl32(1/448)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
@pytest.mark.parametrize("pow2", [False, True])
def test_cast_matches_library_route(fmt, pow2):
    """The cast's encoding step equals torch's float8 conversion of the scaled values."""
    xb = W.normal_bf16(np.random.SeedSequence(11), (64, 1024), 0.7)
    q, s = oracle.cast_per_token(xb, fmt, pow2)
    x = torch.from_numpy(W.bf16_bits_to_f32(xb)).view(64, 8, 128)
    amax = x.abs().amax(-1, keepdim=True).clamp_min(2.0 ** -100)
    fmax = oracle.fp8_max(fmt)
    if pow2:
        mult = 1.0 / torch.from_numpy(s).view(64, 8, 1)
        # s is the smallest power of two with fmax * s >= amax
        sd = torch.from_numpy(s).double().view(64, 8, 1)
        assert torch.all(torch.log2(sd) == torch.round(torch.log2(sd)))
        assert torch.all(fmax * sd >= amax.double()) and torch.all(fmax * sd / 2 < amax.double())
    else:
        mult = torch.tensor(fmax, dtype=torch.float32) / amax
        assert torch.equal(torch.from_numpy(s).view(64, 8, 1), amax / torch.tensor(fmax, dtype=torch.float32))
    ref = (x * mult).to(FMTS[fmt]).view(torch.uint8).view(64, 1024).numpy()
    assert np.array_equal(q, ref)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_cast_invariants(fmt):
    fmax = oracle.fp8_max(fmt)
    xb = W.normal_bf16(np.random.SeedSequence(12), (32, 512), 3e-3)
    xb[3, 128:256] = 0                      # an all-zero group
    q, s = oracle.cast_per_token(xb, fmt)
    x = W.bf16_bits_to_f32(xb).astype(np.float64).reshape(32, 4, 128)
    deq = torch_decode(q, fmt).reshape(32, 4, 128)
    # the element of largest magnitude lands on +-FP8_MAX
    idx = np.abs(x).argmax(-1)
    top = np.take_along_axis(deq, idx[..., None], -1)[..., 0]
    nz = np.abs(x).max(-1) > 0
    assert np.all(np.abs(top[nz]) == fmax)
    # zero group: codes 0, scale at the 2^-100 floor
    assert (q[3, 128:256] == 0).all() and s[3, 1] == np.float32(2.0 ** -100) / np.float32(fmax)
    # reconstruction within half an fp8 spacing (relative 2^-4 for e4m3, 2^-3 for e5m2) plus subnormal floor
    mant = 3 if fmt == oracle.E4M3 else 2
    sub = 2.0 ** (-9 if fmt == oracle.E4M3 else -16)
    err = np.abs(deq * s[..., None] - x)
    bound = (np.abs(x) * 2.0 ** -(mant + 1) * 1.0001 + sub / 2 * s[..., None])
    assert np.all(err <= bound)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
@pytest.mark.parametrize("pow2", [False, True])
def test_cast_f32_matches_library_route_and_bf16_cast(fmt, pow2):
    """The fp32-input cast (of a GEMM epilogue's fp32 result): torch's float8 conversion of the
    values times FP8_MAX / amax, scales amax / FP8_MAX; on bf16-representable inputs it equals the
    bf16 cast."""
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((48, 512)) * 10.0 ** rng.uniform(-3, 3, (48, 1))).astype(np.float32)
    q, s = oracle.cast_per_token_f32(x, fmt, pow2)
    t = torch.from_numpy(x).view(48, 4, 128)
    amax = t.abs().amax(-1, keepdim=True).clamp_min(2.0 ** -100)
    fmax = torch.tensor(oracle.fp8_max(fmt), dtype=torch.float32)
    if pow2:
        sd = torch.from_numpy(s).double().view(48, 4, 1)
        assert torch.all(torch.log2(sd) == torch.round(torch.log2(sd)))
        assert torch.all(fmax * sd >= amax.double()) and torch.all(fmax * sd / 2 < amax.double())
        mult = 1.0 / torch.from_numpy(s).view(48, 4, 1)
    else:
        assert torch.equal(torch.from_numpy(s).view(48, 4, 1), amax / fmax)
        mult = fmax / amax
    ref = (t * mult).to(FMTS[fmt]).view(torch.uint8).view(48, 512).numpy()
    assert np.array_equal(q, ref)
    xb = W.normal_bf16(np.random.SeedSequence(14), (16, 256), 0.4)
    qa, sa = oracle.cast_per_token(xb, fmt, pow2)
    qb, sb = oracle.cast_per_token_f32(W.bf16_bits_to_f32(xb), fmt, pow2)
    assert np.array_equal(qa, qb) and np.array_equal(sa, sb)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_cast_transpose_groups_run_down_the_columns(fmt):
    """The transposed cast groups 128 consecutive rows of one column (the weight gradient's
    contraction over tokens): its scale of (column c, row block rb) is that column segment's
    amax / FP8_MAX, the segment's largest element lands on +-FP8_MAX, and the codes equal
    torch's float8 conversion of the column segment times FP8_MAX / amax."""
    rows, cols = 256, 384
    xb = W.normal_bf16(np.random.SeedSequence(21), (rows, cols), 0.5)
    xb[128:, 7] = 0                                  # an all-zero column segment
    q, s, qt, st = oracle.cast_per_token_transpose(xb, fmt)
    q1, s1 = oracle.cast_per_token(xb, fmt)
    assert np.array_equal(q, q1) and np.array_equal(s, s1)
    assert qt.shape == (cols, rows) and st.shape == (cols, rows // 128)
    x = torch.from_numpy(W.bf16_bits_to_f32(xb))                       # [rows, cols]
    seg = x.view(rows // 128, 128, cols).permute(2, 0, 1)               # [cols, row block, 128 rows]
    amax = seg.abs().amax(-1, keepdim=True).clamp_min(2.0 ** -100)
    fmax = torch.tensor(oracle.fp8_max(fmt), dtype=torch.float32)
    assert torch.equal(torch.from_numpy(st).view(cols, rows // 128, 1), amax / fmax)
    ref = (seg * (fmax / amax)).to(FMTS[fmt]).view(torch.uint8).reshape(cols, rows).numpy()
    assert np.array_equal(qt, ref)
    deq = torch_decode(qt, fmt).reshape(cols, rows // 128, 128)
    top = np.take_along_axis(deq, seg.abs().argmax(-1, keepdim=True).numpy(), -1)[..., 0]
    nz = seg.abs().amax(-1).numpy() > 0
    assert np.all(np.abs(top[nz]) == float(fmax)) and (qt[7, 128:] == 0).all()


def test_operand_row_sums_ones_example_and_brute_force():
    """The pages' all-ones operand: every code is 448 with scale fl32(1/448), so each row sums to
    K * 448 * fl32(1/448); and a brute-force double loop on random codes."""
    q, s = oracle.cast_per_token(bits(np.ones((3, 512))), oracle.E4M3)
    r, mag = oracle.operand_row_sums(q, s, oracle.E4M3)
    want = 512 * 448.0 * float(np.float32(1.0 / 448.0))
    assert np.all(r == want) and np.all(mag == want)
    rng = np.random.default_rng(5)
    q = rng.integers(0, 256, (4, 256), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0                           # no NaN codes
    s = rng.uniform(0.5, 2.0, (4, 2)).astype(np.float32)
    r, _ = oracle.operand_row_sums(q, s, oracle.E4M3)
    for i in range(4):
        acc = 0.0
        for k in range(256):
            acc += float(oracle.decode(q[i:i + 1, k:k + 1], oracle.E4M3)[0, 0]) * float(s[i, k // 128])
        assert abs(acc - r[i]) <= 1e-12 * max(1.0, abs(acc))


def test_cast_rejects_non_finite():
    xb = bits(np.ones((1, 128)))
    xb[0, 5] = 0x7F80  # +inf
    with pytest.raises(ValueError):
        oracle.cast_per_token(xb, oracle.E4M3)


# ------------------------------------------------------------------ GEMM
def random_operand(rng, rows, K, fmt):
    codes = rng.integers(0, 256, size=(rows, K), dtype=np.uint8)
    vals = oracle.decode(np.arange(256, dtype=np.uint8), fmt)
    bad = ~np.isfinite(vals)
    codes[bad[codes]] = 0x38 if fmt == oracle.E4M3 else 0x3C
    scales = rng.uniform(0.25, 4.0, size=(rows, K // 128)).astype(np.float32)
    return codes, scales


@pytest.mark.parametrize("fa,fb", [(oracle.E4M3, oracle.E4M3), (oracle.E5M2, oracle.E4M3),
                                   (oracle.E4M3, oracle.E5M2), (oracle.E5M2, oracle.E5M2)])
@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (3, 2, 256), (2, 3, 128), (37, 19, 512)])
def test_gemm_matches_library_matmul(fa, fb, M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K + fa * 3 + fb)
    qa, sa = random_operand(rng, M, K, fa)
    qb, sb = random_operand(rng, N, K, fb)
    o, d = oracle.gemm_nt(qa, sa, fa, qb, sb, fb)
    A, B = dequant(qa, sa, fa), dequant(qb, sb, fb)
    ref = A @ B.T
    refmag = np.abs(A) @ np.abs(B).T
    assert o.shape == (M, N)
    assert np.allclose(o, ref, rtol=0, atol=1e-12 * refmag.max())
    assert np.allclose(d, refmag, rtol=1e-12)
    # entries form agrees with the full form
    mi = rng.integers(0, M, 10); ni = rng.integers(0, N, 10)
    oe, de = oracle.gemm_nt_entries(qa, sa, fa, qb, sb, fb, mi, ni)
    assert np.array_equal(oe, o[mi, ni]) and np.array_equal(de, d[mi, ni])


def test_gemm_one_hot_identity():
    K = 128
    qa = np.zeros((5, K), np.uint8); qb = np.zeros((7, K), np.uint8)
    for i in range(5):
        qa[i, i * 3] = 0x38      # 1.0
    for j in range(7):
        qb[j, j * 3] = 0x38
    sa = np.arange(1, 6, dtype=np.float32)[:, None] * 0.5
    sb = np.arange(1, 8, dtype=np.float32)[:, None] * 0.25
    o, _ = oracle.gemm_nt(qa, sa, oracle.E4M3, qb, sb, oracle.E4M3)
    want = np.zeros((5, 7))
    for i in range(5):
        want[i, i] = sa[i, 0] * sb[i, 0]
    assert np.array_equal(o, want)


def test_gemm_pow2_scale_linearity():
    rng = np.random.default_rng(3)
    qa, sa = random_operand(rng, 6, 384, oracle.E4M3)
    qb, sb = random_operand(rng, 5, 384, oracle.E4M3)
    o, _ = oracle.gemm_nt(qa, sa, oracle.E4M3, qb, sb, oracle.E4M3)
    o2, _ = oracle.gemm_nt(qa, sa * np.float32(8.0), oracle.E4M3, qb, sb, oracle.E4M3)
    assert np.array_equal(o2, o * 8.0)
    sa3 = sa.copy(); sa3[:, 1] *= np.float32(0.5)  # one K-block only: changes only its term
    o3, _ = oracle.gemm_nt(qa, sa3, oracle.E4M3, qb, sb, oracle.E4M3)
    ob, _ = oracle.gemm_nt(qa, sa, oracle.E4M3, qb, sb, oracle.E4M3, k0=128, K=128)
    assert np.allclose(o3, o - 0.5 * ob, rtol=1e-13, atol=1e-10)


def _ones_example(m, n, k):
    x = bits(np.ones((m, k)))
    y = W.uniform_bf16(np.random.SeedSequence(95), (n, k))
    qx, sx = oracle.cast_per_token(x, oracle.E4M3)
    qy, sy = oracle.cast_per_token(y, oracle.E4M3)
    ref = W.bf16_bits_to_f32(x).astype(np.float32) @ W.bf16_bits_to_f32(y).astype(np.float32).T
    o, d = oracle.gemm_nt(qx, sx, oracle.E4M3, qy, sy, oracle.E4M3)
    return ref, o, d, W.bf16_bits_to_f32(y).astype(np.float64).sum(1)


def test_wgrad_pages_ones_example_doubles():
    """out1 = ref.clone(); out1 += x @ y^T gives out1/ref near 2 (printed 1.9995 .. 2.0009)."""
    with open(os.path.join(GOLD, "wgrad_ones_example.txt")) as f:
        kv = {l.split()[0]: l.split()[1:] for l in f if l.strip() and not l.startswith("#")}
    k = int(kv["k"][0]); n = int(kv["n"][0])
    printed = np.array([float(v) for v in kv["printed_ratios"]])
    assert printed.min() >= 1.999 and printed.max() <= 2.001
    ref, o, d, rowsum = _ones_example(4, n, k)
    out1, _ = oracle.wgrad(o, d, ref)
    ratio = out1 / ref
    assert np.all(np.abs(ratio - 2.0) < 2e-3), (ratio.min(), ratio.max())
    # zero-initialised out: close to ref, and to the bf16 row sums of y
    out0, _ = oracle.wgrad(o, d, np.zeros_like(ref))
    assert np.all(np.abs(out0 / ref - 1.0) < 2e-3)
    assert np.all(np.abs(out0[0] / rowsum - 1.0) < 2e-3)


def test_wgrad_second_call_doubles():
    rng = np.random.default_rng(5)
    qa, sa = random_operand(rng, 9, 256, oracle.E4M3)
    qb, sb = random_operand(rng, 4, 256, oracle.E4M3)
    o, d = oracle.gemm_nt(qa, sa, oracle.E4M3, qb, sb, oracle.E4M3)
    first, _ = oracle.wgrad(o, d, np.zeros((9, 4), np.float32))
    second, _ = oracle.wgrad(o, d, first.astype(np.float32))
    assert np.allclose(second, 2 * first, rtol=1e-7)
    init = rng.standard_normal((9, 4)).astype(np.float32)
    got, mag = oracle.wgrad(o, d, init)
    assert np.array_equal(got, init.astype(np.float64) + o)
    assert np.array_equal(mag, np.abs(init.astype(np.float64)) + d)


# ------------------------------------------------------------- epilogues
def test_gelu_matches_torch_tanh_gelu_and_its_gradient():
    z = torch.linspace(-12, 12, 2001, dtype=torch.float64, requires_grad=True)
    g = torch.nn.functional.gelu(z, approximate="tanh")
    (dg,) = torch.autograd.grad(g.sum(), z)
    ours = np.array([oracle.gelu(v) for v in z.detach().numpy()])
    dours = np.array([oracle.dgelu(v) for v in z.detach().numpy()])
    assert np.allclose(ours, g.detach().numpy(), rtol=1e-14, atol=1e-15)
    assert np.allclose(dours, dg.numpy(), rtol=1e-12, atol=1e-14)
    assert oracle.gelu(0.0) == 0.0 and oracle.dgelu(0.0) == 0.5
    assert abs(oracle.gelu(40.0) - 40.0) < 1e-12 and abs(oracle.gelu(-40.0)) < 1e-12


def test_fwd_bias_broadcasts_down_columns():
    """X = 0 and b != 0: Y = GELU(b[n]) in every row (b has length n, the output features)."""
    M, N, K = 3, 5, 128
    qx = np.zeros((M, K), np.uint8); sx = np.ones((M, 1), np.float32)
    rng = np.random.default_rng(1)
    qw, sw = random_operand(rng, N, K, oracle.E4M3)
    o, d = oracle.gemm_nt(qx, sx, oracle.E4M3, qw, sw, oracle.E4M3)
    b = bits(np.array([-1.5, -0.25, 0.0, 0.5, 2.0]))
    y, z, zmag = oracle.fwd_epilogue(o, d, b, gelu_on=True)
    bref = torch.from_numpy(W.bf16_bits_to_f32(b).astype(np.float64))
    want = torch.nn.functional.gelu(bref, approximate="tanh").numpy()
    for m in range(M):
        assert np.allclose(y[m], want, rtol=1e-14, atol=1e-16)
        assert np.array_equal(z[m], W.bf16_bits_to_f32(b).astype(np.float64))
    y2, _, _ = oracle.fwd_epilogue(o, d, b, gelu_on=False)
    assert np.array_equal(y2, z)


def test_fwd_matches_library_linear():
    rng = np.random.default_rng(2)
    qx, sx = random_operand(rng, 6, 256, oracle.E4M3)
    qw, sw = random_operand(rng, 4, 256, oracle.E4M3)
    b = W.normal_bf16(np.random.SeedSequence(3), (4,), 0.1)
    o, d = oracle.gemm_nt(qx, sx, oracle.E4M3, qw, sw, oracle.E4M3)
    y, _, _ = oracle.fwd_epilogue(o, d, b, gelu_on=True)
    X = torch.from_numpy(dequant(qx, sx, oracle.E4M3))
    Wt = torch.from_numpy(dequant(qw, sw, oracle.E4M3))
    bt = torch.from_numpy(W.bf16_bits_to_f32(b).astype(np.float64))
    ref = torch.nn.functional.gelu(torch.nn.functional.linear(X, Wt, bt), approximate="tanh")
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


def _dgrad_case(zval):
    rng = np.random.default_rng(4)
    qa, sa = random_operand(rng, 8, 256, oracle.E5M2)
    qb, sb = random_operand(rng, 6, 256, oracle.E4M3)
    o, d = oracle.gemm_nt(qa, sa, oracle.E5M2, qb, sb, oracle.E4M3)
    z = bits(np.full((8, 6), zval))
    return o, d, z


def test_dgrad_order_dgelu_before_bias_grad():
    o, d, z = _dgrad_case(0.0)
    D, _, db, _ = oracle.dgrad_epilogue(o, d, z, bgrad=True)
    assert np.array_equal(D, 0.5 * o)                      # GELU'(0) = 1/2 exactly
    assert np.allclose(db, 0.5 * o.sum(axis=0), rtol=1e-14)
    o, d, z = _dgrad_case(30.0)                            # GELU'(z) -> 1
    _, _, db, _ = oracle.dgrad_epilogue(o, d, z, bgrad=True)
    assert np.allclose(db, o.sum(axis=0), rtol=1e-12)
    o, d, z = _dgrad_case(-30.0)                           # GELU'(z) -> 0
    _, _, db, _ = oracle.dgrad_epilogue(o, d, z, bgrad=True)
    assert np.all(np.abs(db) < 1e-100 * np.abs(o).sum(axis=0) + 1e-300)


def test_dgrad_matches_autograd_of_library_linear():
    """dZ and db from torch autograd through y = gelu(z), z = x W^T + b, at the same dY."""
    rng = np.random.default_rng(6)
    M, N, K = 7, 5, 256                                     # D is [M, N], contraction K
    qa, sa = random_operand(rng, M, K, oracle.E5M2)
    qb, sb = random_operand(rng, N, K, oracle.E4M3)
    zb = W.normal_bf16(np.random.SeedSequence(8), (M, N), 1.3)
    o, d = oracle.gemm_nt(qa, sa, oracle.E5M2, qb, sb, oracle.E4M3)
    D, _, db, _ = oracle.dgrad_epilogue(o, d, zb, bgrad=True)
    zt = torch.from_numpy(W.bf16_bits_to_f32(zb).astype(np.float64)).requires_grad_(True)
    bias = torch.zeros(N, dtype=torch.float64, requires_grad=True)
    y = torch.nn.functional.gelu(zt + bias, approximate="tanh")
    dy = torch.from_numpy(dequant(qa, sa, oracle.E5M2) @ dequant(qb, sb, oracle.E4M3).T)
    gz, gb = torch.autograd.grad(y, (zt, bias), dy)
    assert np.allclose(D, gz.numpy(), rtol=1e-11, atol=1e-12 * np.abs(D).max())
    assert db.shape == (N,)
    assert np.allclose(db, gb.numpy(), rtol=1e-11, atol=1e-12 * np.abs(db).max())


def test_dgrad_without_epilogue_is_plain_product():
    o, d, _ = _dgrad_case(0.0)
    D, Dm, db, _ = oracle.dgrad_epilogue(o, d, None, bgrad=False)
    assert np.array_equal(D, o) and np.array_equal(Dm, d) and db is None


# ------------------------------------------------------------- K-grouped
def test_kgrouped_equals_dense_per_group_and_skips_empty():
    rng = np.random.default_rng(9)
    gk = np.array([256, 0, 128, 384, 0], np.int64)
    M, N, S = 6, 5, int(gk.sum())
    qa, sa = random_operand(rng, M, S, oracle.E4M3)
    qb, sb = random_operand(rng, N, S, oracle.E4M3)
    init = rng.standard_normal((5, M, N)).astype(np.float32)
    out, mag = oracle.kgrouped_wgrad(qa, sa, oracle.E4M3, qb, sb, oracle.E4M3, gk, init)
    A, B = dequant(qa, sa, oracle.E4M3), dequant(qb, sb, oracle.E4M3)
    off = 0
    for g, k in enumerate(gk):
        want = init[g].astype(np.float64) + A[:, off:off + k] @ B[:, off:off + k].T
        assert np.allclose(out[g], want, rtol=1e-12, atol=1e-12)
        if k == 0:
            assert np.array_equal(out[g], init[g].astype(np.float64))
        off += k
    # group order does not matter: permuting groups (and their column slices) permutes outputs
    perm = [3, 0, 4, 2, 1]
    offs = np.concatenate([[0], np.cumsum(gk)])
    cols = np.concatenate([np.arange(offs[g], offs[g + 1]) for g in perm]).astype(np.int64)
    blocks = np.concatenate([np.arange(offs[g] // 128, offs[g + 1] // 128) for g in perm]).astype(np.int64)
    out_p, _ = oracle.kgrouped_wgrad(qa[:, cols], sa[:, blocks], oracle.E4M3, qb[:, cols], sb[:, blocks],
                                     oracle.E4M3, gk[perm], init[perm])
    assert np.allclose(out_p, out[perm], rtol=1e-14, atol=1e-14)


# ------------------------------------------------------------- M-grouped
def _mgrouped_case(seed, G, nblocks, N, K, block=8, fx=oracle.E4M3):
    """Random codes with `block`-row blocks (the oracle's block size is a parameter; the library's
    is 256 rows, which changes nothing in the definition)."""
    rng = np.random.default_rng(seed)
    qx, sx = random_operand(rng, nblocks * block, K, fx)
    ws = [random_operand(rng, N, K, oracle.E4M3) for _ in range(G)]
    qw, sw = np.stack([w[0] for w in ws]), np.stack([w[1] for w in ws])
    b = W.normal_bf16(np.random.SeedSequence(seed + 1), (G, N), 0.1)
    z = W.normal_bf16(np.random.SeedSequence(seed + 2), (nblocks * block, N), 1.3)
    return qx, sx, qw, sw, b, z


def test_mgrouped_fwd_one_expert_is_the_dense_forward():
    """Every block on expert e: the dense forward with W[e] and bias[e] over the whole matrix."""
    qx, sx, qw, sw, b, _ = _mgrouped_case(11, 3, 4, 6, 256)
    for e in range(3):
        y, z, zm = oracle.mgrouped_fwd(qx, sx, oracle.E4M3, qw, sw, oracle.E4M3, np.full(4, e), b, True, block=8)
        o, d = oracle.gemm_nt(qx, sx, oracle.E4M3, qw[e], sw[e], oracle.E4M3)
        yd, zd, zmd = oracle.fwd_epilogue(o, d, b[e], True)
        assert np.array_equal(y, yd) and np.array_equal(z, zd) and np.array_equal(zm, zmd)


def test_mgrouped_fwd_brute_force_and_block_permutation():
    """Per-block library Linear (torch decode, matmul, tanh-GELU) with each block's own expert; skipped
    blocks stay NaN; permuting the blocks (rows and expert list together) permutes the output rows."""
    blocks = np.array([2, -1, 0, 2, 1])
    qx, sx, qw, sw, b, _ = _mgrouped_case(12, 3, len(blocks), 5, 384)
    y, _, _ = oracle.mgrouped_fwd(qx, sx, oracle.E4M3, qw, sw, oracle.E4M3, blocks, b, True, block=8)
    X = torch.from_numpy(dequant(qx, sx, oracle.E4M3))
    for i, e in enumerate(blocks):
        r = slice(8 * i, 8 * (i + 1))
        if e < 0:
            assert np.isnan(y[r]).all()
            continue
        Wt = torch.from_numpy(dequant(qw[e], sw[e], oracle.E4M3))
        bt = torch.from_numpy(W.bf16_bits_to_f32(b[e]).astype(np.float64))
        ref = torch.nn.functional.gelu(torch.nn.functional.linear(X[r], Wt, bt), approximate="tanh")
        assert np.allclose(y[r], ref.numpy(), rtol=1e-12, atol=1e-12)
    perm = np.array([3, 0, 4, 1, 2])
    rows = np.concatenate([np.arange(8 * p, 8 * p + 8) for p in perm])
    yp, _, _ = oracle.mgrouped_fwd(qx[rows], sx[rows], oracle.E4M3, qw, sw, oracle.E4M3, blocks[perm], b, True,
                                   block=8)
    assert np.array_equal(yp, y[rows], equal_nan=True)


def test_mgrouped_dgrad_one_expert_is_the_dense_dgrad():
    """Every block on expert e: D and the bias gradient of the dense dgrad over the whole matrix; the
    other experts' bias gradients are zero."""
    qa, sa, qw, sw, _, z = _mgrouped_case(13, 3, 4, 6, 256)
    D, Dm, db, dbm = oracle.mgrouped_dgrad(qa, sa, oracle.E4M3, qw, sw, oracle.E4M3, np.full(4, 1), z, block=8)
    o, d = oracle.gemm_nt(qa, sa, oracle.E4M3, qw[1], sw[1], oracle.E4M3)
    Dd, Dmd, dbd, dbmd = oracle.dgrad_epilogue(o, d, z, bgrad=True)
    assert np.array_equal(D, Dd) and np.array_equal(Dm, Dmd)
    assert np.allclose(db[1], dbd, rtol=1e-13, atol=1e-13 * dbmd.max())
    assert np.allclose(dbm[1], dbmd, rtol=1e-13)
    assert (db[0] == 0).all() and (db[2] == 0).all()


def test_mgrouped_dgrad_brute_force_skips_and_per_expert_sums():
    """Library route per block (torch decode, matmul, autograd of the tanh-GELU); a -1 block is
    neither written nor summed; expert e's bias gradient is the column sum over its blocks' rows;
    permuting the blocks permutes the rows and leaves the bias gradients unchanged."""
    blocks = np.array([1, 0, -1, 1, 2])
    G, N, K = 4, 5, 256
    qa, sa, qw, sw, _, z = _mgrouped_case(14, G, len(blocks), N, K, fx=oracle.E5M2)
    D, _, db, _ = oracle.mgrouped_dgrad(qa, sa, oracle.E5M2, qw, sw, oracle.E4M3, blocks, z, block=8)
    A = dequant(qa, sa, oracle.E5M2)
    want_db = np.zeros((G, N))
    for i, e in enumerate(blocks):
        r = slice(8 * i, 8 * (i + 1))
        if e < 0:
            assert np.isnan(D[r]).all()
            continue
        dy = torch.from_numpy(A[r] @ dequant(qw[e], sw[e], oracle.E4M3).T)
        zt = torch.from_numpy(W.bf16_bits_to_f32(z[r]).astype(np.float64)).requires_grad_(True)
        (gz,) = torch.autograd.grad(torch.nn.functional.gelu(zt, approximate="tanh"), zt, dy)
        assert np.allclose(D[r], gz.numpy(), rtol=1e-11, atol=1e-12 * np.abs(gz.numpy()).max())
        want_db[e] += gz.numpy().sum(0)
    assert np.allclose(db, want_db, rtol=1e-11, atol=1e-12 * np.abs(want_db).max())
    assert (db[3] == 0).all()
    live = ~np.isnan(D[:, 0])
    for e in range(G):
        rows_e = np.repeat(blocks == e, 8)
        assert np.allclose(db[e], D[rows_e & live].sum(0), rtol=1e-12, atol=1e-13)
    perm = np.array([4, 2, 0, 3, 1])
    rows = np.concatenate([np.arange(8 * p, 8 * p + 8) for p in perm])
    Dp, _, dbp, _ = oracle.mgrouped_dgrad(qa[rows], sa[rows], oracle.E5M2, qw, sw, oracle.E4M3, blocks[perm],
                                          z[rows], block=8)
    assert np.array_equal(Dp, D[rows], equal_nan=True)
    assert np.allclose(dbp, db, rtol=1e-13, atol=1e-13 * np.abs(db).max())
