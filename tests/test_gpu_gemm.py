"""GPU parity of the four GEMM entry points against the fp64 oracle.

The oracle casts the seeded bf16 inputs on the host; those fp8 bytes and
scales are uploaded and consumed by the HIP kernels, so both sides see the
same operands (the cast kernel has its own bit-exact test).  Small cases span
several 256 x 256 tiles with ragged edges and are compared element by element;
the workload sizes are compared on a sampled grid of rows x columns that
includes the first and last rows/columns and tile boundaries.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import (BIAS_CHAIN, GELU_CHAIN, GELU_LIP, bf16_dev, bf16_host_f64, chain_colsum, chain_gemm, chain_rowsum,
                    check_bf16, check_f32, check_quant, dev, host, scale_ld, sdev, shost)

te = pytest.importorskip("fp8_linear_layer_amd")
pytestmark = pytest.mark.gpu

E4, E5 = te.TE_DTYPE_E4M3, te.TE_DTYPE_E5M2
OF = {E4: oracle.E4M3, E5: oracle.E5M2}
FULL, FAST = te.TE_ACCUM_FULL_FP32, te.TE_ACCUM_FAST
POLICIES = [(FULL, False), (FAST, False), (FAST, True)]  # (accum, pow2-scaled inputs)
PID = ["full", "fast", "fast-pow2"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    te.load_library()


def epi_chain(epi):
    """Extra fp32 roundings of an epilogue (bias add, GELU or GELU')."""
    return (BIAS_CHAIN if epi & te.TE_EPI_BIAS else 0) + \
        (GELU_CHAIN if epi & (te.TE_EPI_GELU | te.TE_EPI_DGELU) else 0)


@pytest.fixture(params=["wave", "persistent"])
def gemm_path(request, monkeypatch):
    """Small products run on both GEMM kernels: the wave-tile one (the library's choice for
    products with few 256 x 256 tiles) and, forced through TE_FP8_GEMM_PATH, the persistent one."""
    monkeypatch.setenv("TE_FP8_GEMM_PATH", request.param)
    return request.param


def operand(seed, rows, K, dt, std=1.0, pow2=False):
    bits = W.normal_bf16(np.random.SeedSequence(seed), (rows, K), std)
    q, s = oracle.cast_per_token(bits, OF[dt], pow2)
    return q, s


def sample_idx(n, k, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, n - 1, n - 2] + [b + d for b in (255, 256, 511, 512, n // 2) for d in (0, 1)]
    idx = np.concatenate([np.array([i for i in fixed if 0 <= i < n]), rng.integers(0, n, k)])
    return np.unique(idx)


def grid_entries(qa, sa, fa, qb, sb, fb, rows, cols, k0=0, K=None):
    mi = np.repeat(rows, len(cols)).astype(np.int64)
    ni = np.tile(cols, len(rows)).astype(np.int64)
    o, d = oracle.gemm_nt_entries(qa, sa, fa, qb, sb, fb, mi, ni, k0, K)
    return o.reshape(len(rows), len(cols)), d.reshape(len(rows), len(cols))


# ------------------------------------------------------------------ wgrad
@pytest.mark.parametrize("accum,pow2", POLICIES, ids=PID)
@pytest.mark.parametrize("da,db", [(E4, E4), (E5, E4), (E4, E5), (E5, E5)])
@pytest.mark.parametrize("M,N,K", [(300, 520, 384), (1, 1, 128), (256, 256, 512), (513, 200, 256)])
def test_wgrad_small(accum, pow2, da, db, M, N, K, gemm_path):
    qa, sa = operand(M * 3 + K, M, K, da, pow2=pow2)
    qb, sb = operand(N * 5 + K + 1, N, K, db, pow2=pow2)
    out0 = W.normal_f32(np.random.SeedSequence(M + N), (M, N))
    o, d = oracle.gemm_nt(qa, sa, OF[da], qb, sb, OF[db])
    want, mag = oracle.wgrad(o, d, out0)
    ld = N + 12 - (N + 12) % 4
    buf = torch.full((M + 1, ld), 1234.5, dtype=torch.float32, device="cuda")
    buf[:M, :N] = dev(out0)
    out = buf[:M, :N]
    te.te_fp8_wgrad_accum(dev(qa), sdev(sa), da, dev(qb), sdev(sb), db, out, accum)
    torch.cuda.synchronize()
    b = host(buf).numpy()
    assert (b[:M, N:] == 1234.5).all() and (b[M:] == 1234.5).all(), "wrote outside out"
    check_f32(b[:M, :N], want, mag, "wgrad", chain_gemm(K, 1))


@pytest.mark.parametrize("accum,pow2", [(FULL, False), (FAST, True)], ids=["full", "fast-pow2"])
def test_wgrad_max_k(accum, pow2):
    """The largest contraction the ABI accepts, K = 2^22 (32768 scale blocks in one tile's loop)."""
    M, N, K = 3, 4, 1 << 22
    qa, sa = operand(101, M, K, E4, pow2=pow2)
    qb, sb = operand(102, N, K, E4, pow2=pow2)
    out0 = W.normal_f32(np.random.SeedSequence(103), (M, N))
    o, d = oracle.gemm_nt(qa, sa, oracle.E4M3, qb, sb, oracle.E4M3)
    want, mag = oracle.wgrad(o, d, out0)
    out = dev(out0)
    te.te_fp8_wgrad_accum(dev(qa), sdev(sa), E4, dev(qb), sdev(sb), E4, out, accum)
    check_f32(host(out).numpy(), want, mag, "wgrad K=2^22", chain_gemm(K, 1))


@pytest.mark.parametrize("da", [E4, E5])
@pytest.mark.parametrize("M,N,K", [(300, 200, 384), (7, 16, 1024), (513, 64, 128)])
def test_wgrad_with_bias_grad(da, M, N, K, gemm_path):
    """out += A B^T exactly as the plain call, plus bias_grad[m] = the dequantised row sums of A."""
    qa, sa = operand(M + K + 7, M, K, da)
    qb, sb = operand(N + K + 8, N, K, E4)
    out0 = W.normal_f32(np.random.SeedSequence(M + 9), (M, N))
    A, SA, B, SB = dev(qa), sdev(sa), dev(qb), sdev(sb)
    ld = N + 4 - N % 4
    out = torch.empty((M, ld), dtype=torch.float32, device="cuda")[:, :N]
    out.copy_(dev(out0))
    ref = torch.empty((M, ld), dtype=torch.float32, device="cuda")[:, :N]
    ref.copy_(dev(out0))
    bg = torch.full((M + 3,), 5.0, dtype=torch.float32, device="cuda")
    te.te_fp8_wgrad_accum_bgrad(A, SA, da, B, SB, E4, out, bg[:M], FULL)
    te.te_fp8_wgrad_accum(A, SA, da, B, SB, E4, ref, FULL)
    assert torch.equal(host(out).view(torch.int32), host(ref).view(torch.int32))
    g = host(bg).numpy()
    assert np.all(g[M:] == 5.0)
    want, mag = oracle.operand_row_sums(qa, sa, OF[da])
    check_f32(g[:M], want, mag, "bias grad from A", chain_rowsum(K), mma=False)


def test_wgrad_pages_ones_example():
    """out1 = ref.clone(); out1 += x y^T makes out1/ref ~ 2; zero-initialised out gives ~ref."""
    m, n, k = 512, 1024, 4096
    x = W.f32_to_bf16_bits(np.ones((m, k), np.float32))
    y = W.uniform_bf16(np.random.SeedSequence(95), (n, k))
    qx, sx = oracle.cast_per_token(x, oracle.E4M3)
    qy, sy = oracle.cast_per_token(y, oracle.E4M3)
    ref = (W.bf16_bits_to_f32(x) @ W.bf16_bits_to_f32(y).T).astype(np.float32)
    out1 = dev(ref)
    te.te_fp8_wgrad_accum(dev(qx), sdev(sx), E4, dev(qy), sdev(sy), E4, out1, FULL)
    r = host(out1).numpy() / ref
    assert np.all(np.abs(r - 2.0) < 2e-3), (r.min(), r.max())
    out0 = torch.zeros((m, n), dtype=torch.float32, device="cuda")
    te.te_fp8_wgrad_accum(dev(qx), sdev(sx), E4, dev(qy), sdev(sy), E4, out0, FULL)
    r0 = host(out0).numpy() / ref
    assert np.all(np.abs(r0 - 1.0) < 2e-3)
    # a second call doubles
    te.te_fp8_wgrad_accum(dev(qx), sdev(sx), E4, dev(qy), sdev(sy), E4, out0, FULL)
    assert np.allclose(host(out0).numpy() / ref, 2 * r0, rtol=1e-6)


@pytest.mark.parametrize("accum", [FULL, FAST])
def test_wgrad_deterministic(accum):
    qa, sa = operand(1, 384, 1024, E4)
    qb, sb = operand(2, 640, 1024, E4)
    outs = []
    for _ in range(2):
        out = torch.zeros((384, 640), dtype=torch.float32, device="cuda")
        te.te_fp8_wgrad_accum(dev(qa), sdev(sa), E4, dev(qb), sdev(sb), E4, out, accum)
        outs.append(host(out).numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


@pytest.mark.parametrize("accum,pow2", [(FULL, False), (FAST, True)], ids=["full", "fast-pow2"])
def test_wgrad_dense_workload(accum, pow2):
    sh = W.DENSE_WGRAD.shapes
    inp = W.dense_wgrad_inputs()
    qa, sa = oracle.cast_per_token(inp["a"], oracle.E4M3, pow2)
    qb, sb = oracle.cast_per_token(inp["b"], oracle.E4M3, pow2)
    out = dev(inp["out0"])
    te.te_fp8_wgrad_accum(dev(qa), sdev(sa), E4, dev(qb), sdev(sb), E4, out, accum)
    got = host(out).numpy()
    rows, cols = sample_idx(sh["M"], 40, 1), sample_idx(sh["N"], 40, 2)
    o, d = grid_entries(qa, sa, oracle.E4M3, qb, sb, oracle.E4M3, rows, cols)
    init = inp["out0"][np.ix_(rows, cols)]
    check_f32(got[np.ix_(rows, cols)], init.astype(np.float64) + o, np.abs(init) + d, "dense wgrad",
              chain_gemm(sh["K"], 1))


# ------------------------------------------------------------------ fprop
FWD_EPIS = [te.TE_EPI_NONE, te.TE_EPI_BIAS, te.TE_EPI_BIAS | te.TE_EPI_GELU,
            te.TE_EPI_BIAS | te.TE_EPI_GELU | te.TE_EPI_AUX_PREACT, te.TE_EPI_GELU]


def fwd_case(M, N, K, epi, ydt, accum, pow2, xs=1.0, ws=1.0, seed=0):
    qx, sx = operand(seed + 11, M, K, E4, xs, pow2)
    qw, sw = operand(seed + 12, N, K, E4, ws, pow2)
    b = W.normal_bf16(np.random.SeedSequence(seed + 13), (N,), 0.1)
    o, d = oracle.gemm_nt(qx, sx, oracle.E4M3, qw, sw, oracle.E4M3)
    has_b = bool(epi & te.TE_EPI_BIAS)
    y, z, zmag = oracle.fwd_epilogue(o, d, b if has_b else None, bool(epi & te.TE_EPI_GELU))
    return qx, sx, qw, sw, b, y, z, zmag


@pytest.mark.parametrize("accum,pow2", POLICIES, ids=PID)
@pytest.mark.parametrize("epi", FWD_EPIS)
@pytest.mark.parametrize("ydt", [te.TE_DTYPE_F32, te.TE_DTYPE_BF16])
@pytest.mark.parametrize("M,N,K", [(300, 264, 512), (17, 36, 128)])
def test_fwd_small(accum, pow2, epi, ydt, M, N, K, gemm_path):
    qx, sx, qw, sw, b, y, z, zmag = fwd_case(M, N, K, epi, ydt, accum, pow2, seed=M)
    ymag = zmag * (GELU_LIP if epi & te.TE_EPI_GELU else 1.0)
    tdt = torch.float32 if ydt == te.TE_DTYPE_F32 else torch.bfloat16
    ld = (N + 8) // 8 * 8
    ybuf = torch.full((M + 1, ld), 77.0, dtype=tdt, device="cuda")
    yv = ybuf[:M, :N]
    pre = None
    if epi & te.TE_EPI_AUX_PREACT:
        prebuf = torch.full((M, ld), 55.0, dtype=torch.bfloat16, device="cuda")
        pre = prebuf[:, :N]
    te.te_fp8_gemm_fwd(dev(qx), sdev(sx), E4, dev(qw), sdev(sw), E4,
                       bias=bf16_dev(b) if epi & te.TE_EPI_BIAS else None, epilogue=epi,
                       y=yv, y_dtype=ydt, preact=pre, accum=accum)
    torch.cuda.synchronize()
    yb = host(ybuf)
    assert torch.all(yb[:M, N:] == 77.0) and torch.all(yb[M:] == 77.0), "wrote outside y"
    if ydt == te.TE_DTYPE_F32:
        check_f32(yb[:M, :N].numpy(), y, ymag, "fwd y", chain_gemm(K, epi_chain(epi)))
    else:
        check_bf16(bf16_host_f64(yb[:M, :N]), y, ymag, "fwd y")
    if pre is not None:
        pb = host(prebuf)
        assert torch.all(pb[:, N:] == 55.0)
        check_bf16(bf16_host_f64(pb[:, :N]), z, zmag, "fwd preact")


def quant_fwd(qx, sx, qw, sw, b, epi, accum, qdt, cast_pow2, M, N, pre=None):
    """Run the quantising forward with sentinel-filled outputs; return (q, row-major scales) and
    check that nothing outside them was written."""
    qbuf = torch.full((M, N + 16), 0xA5, dtype=torch.uint8, device="cuda")
    qs = torch.full((N // 128, scale_ld(M)), -3.0, dtype=torch.float32, device="cuda")
    te.te_fp8_gemm_fwd_quant(dev(qx), sdev(sx), E4, dev(qw), sdev(sw), E4,
                             bias=bf16_dev(b) if epi & te.TE_EPI_BIAS else None, epilogue=epi, q_dtype=qdt,
                             cast_flags=te.TE_CAST_POW2_SCALE if cast_pow2 else 0, q=qbuf[:, :N], q_scales=qs,
                             preact=pre, accum=accum)
    torch.cuda.synchronize()
    qh, sh = host(qbuf).numpy(), host(qs).numpy()
    assert (qh[:, N:] == 0xA5).all(), "wrote past N"
    assert (sh[:, M:] == -3.0).all(), "wrote into the scale padding"
    return qh[:, :N], shost(qs, M)


@pytest.mark.parametrize("accum,pow2", POLICIES, ids=PID)
@pytest.mark.parametrize("epi", FWD_EPIS)
@pytest.mark.parametrize("qdt,cast_pow2", [(te.TE_DTYPE_E4M3, False), (te.TE_DTYPE_E5M2, False),
                                           (te.TE_DTYPE_E4M3, True)])
@pytest.mark.parametrize("M,N,K", [(300, 384, 512), (17, 128, 128)])
def test_fwd_quant(accum, pow2, epi, qdt, cast_pow2, M, N, K, gemm_path):
    """The quantised forward equals the per-token cast of the forward's own fp32 result (the oracle's
    fp32-input cast of the fp32 y the plain forward call returns: the codes are decided in the
    kernel's fp32), and that fp32 y matches the fp64 oracle."""
    qx, sx, qw, sw, b, y, z, zmag = fwd_case(M, N, K, epi, te.TE_DTYPE_F32, accum, pow2, seed=M + 5)
    y32 = te.te_fp8_gemm_fwd(dev(qx), sdev(sx), E4, dev(qw), sdev(sw), E4,
                             bias=bf16_dev(b) if epi & te.TE_EPI_BIAS else None, epilogue=epi & ~te.TE_EPI_AUX_PREACT,
                             y_dtype=te.TE_DTYPE_F32, accum=accum)
    y32h = host(y32).numpy()
    check_f32(y32h, y, zmag * (GELU_LIP if epi & te.TE_EPI_GELU else 1.0), "fwd y (fp32)",
              chain_gemm(K, epi_chain(epi)))
    pre = None
    if epi & te.TE_EPI_AUX_PREACT:
        prebuf = torch.full((M, N + 8), 55.0, dtype=torch.bfloat16, device="cuda")
        pre = prebuf[:, :N]
    q, s = quant_fwd(qx, sx, qw, sw, b, epi, accum, qdt, cast_pow2, M, N, pre)
    qo, so = oracle.cast_per_token_f32(y32h, OF[qdt], cast_pow2)
    bad = np.argwhere(q != qo)
    assert bad.size == 0, f"{len(bad)} code mismatches, first {bad[0]}"
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32)), "scale mismatch"
    # and the dequantised store against the fp64 oracle
    check_quant(q, s, OF[qdt], y, zmag * (GELU_LIP if epi & te.TE_EPI_GELU else 1.0), "fwd quant vs oracle",
                chain_gemm(K, epi_chain(epi)))
    if pre is not None:
        pb = host(prebuf)
        assert torch.all(pb[:, N:] == 55.0)
        check_bf16(bf16_host_f64(pb[:, :N]), z, zmag, "fwd preact")


def quant_t_bufs(M, N):
    """Sentinel-filled transposed-cast outputs (qt with 16 padding columns, the scale padding)."""
    qt = torch.full((N, M + 16), 0x5A, dtype=torch.uint8, device="cuda")
    qts = torch.full((M // 128, scale_ld(N)), -7.0, dtype=torch.float32, device="cuda")
    return qt, qts


def check_quant_t(qt, qts, M, N, y32h, y, ymag, fmt, cast_pow2, chain, what):
    """The transposed cast: bit-exact against the oracle's cast of the kernel's own fp32 result's
    transpose, held to the fp64 oracle, and nothing written outside it."""
    qth, qtsh = host(qt).numpy(), host(qts).numpy()
    assert (qth[:, M:] == 0x5A).all(), f"{what}: wrote past M"
    assert (qtsh[:, N:] == -7.0).all(), f"{what}: wrote into the scale padding"
    qo, so = oracle.cast_per_token_f32(np.ascontiguousarray(y32h.T), fmt, cast_pow2)
    bad = np.argwhere(qth[:, :M] != qo)
    assert bad.size == 0, f"{what}: {len(bad)} transposed code mismatches, first {bad[0]}"
    st = shost(qts, N)
    assert np.array_equal(st.view(np.uint32), so.view(np.uint32)), f"{what}: transposed scale mismatch"
    check_quant(qth[:, :M], st, fmt, y.T, ymag.T, what + " vs oracle", chain)


@pytest.mark.parametrize("accum,pow2", POLICIES, ids=PID)
@pytest.mark.parametrize("epi", [te.TE_EPI_NONE, te.TE_EPI_BIAS | te.TE_EPI_GELU])
@pytest.mark.parametrize("qdt,cast_pow2", [(te.TE_DTYPE_E4M3, False), (te.TE_DTYPE_E5M2, True)])
@pytest.mark.parametrize("M,N,K", [(384, 384, 512), (128, 128, 128), (640, 256, 256)])
def test_fwd_quant_transposed(accum, pow2, epi, qdt, cast_pow2, M, N, K):
    """Both casts of the forward's fp32 result from one call: the row-wise one bit-identical to the
    row-wise-only call, the transposed one (groups of 128 rows) to the oracle's cast of y^T; the
    transposed-only call gives the same bytes."""
    qx, sx, qw, sw, b, y, z, zmag = fwd_case(M, N, K, epi, te.TE_DTYPE_F32, accum, pow2, seed=M + 9)
    ymag = zmag * (GELU_LIP if epi & te.TE_EPI_GELU else 1.0)
    X, SX, Wd, SW = dev(qx), sdev(sx), dev(qw), sdev(sw)
    B = bf16_dev(b) if epi & te.TE_EPI_BIAS else None
    cf = te.TE_CAST_POW2_SCALE if cast_pow2 else 0
    y32h = host(te.te_fp8_gemm_fwd(X, SX, E4, Wd, SW, E4, bias=B, epilogue=epi, y_dtype=te.TE_DTYPE_F32,
                                   accum=accum)).numpy()
    q1, s1 = te.te_fp8_gemm_fwd_quant(X, SX, E4, Wd, SW, E4, bias=B, epilogue=epi, q_dtype=qdt, cast_flags=cf,
                                      accum=accum)
    qt, qts = quant_t_bufs(M, N)
    q2, s2, _, _ = te.te_fp8_gemm_fwd_quant(X, SX, E4, Wd, SW, E4, bias=B, epilogue=epi, q_dtype=qdt, cast_flags=cf,
                                            accum=accum, transposed=True, qt=qt[:, :M], qt_scales=qts)
    torch.cuda.synchronize()
    assert torch.equal(host(q1), host(q2)) and torch.equal(host(s1).view(torch.int32), host(s2).view(torch.int32))
    chain = chain_gemm(K, epi_chain(epi))
    check_quant_t(qt, qts, M, N, y32h, y, ymag, OF[qdt], cast_pow2, chain, "fwd qt")
    qt3, qts3 = quant_t_bufs(M, N)
    te.te_fp8_gemm_fwd_quant(X, SX, E4, Wd, SW, E4, bias=B, epilogue=epi, q_dtype=qdt, cast_flags=cf, accum=accum,
                             rowwise=False, transposed=True, qt=qt3[:, :M], qt_scales=qts3)
    assert torch.equal(host(qt3), host(qt)) and torch.equal(host(qts3).view(torch.int32), host(qts).view(torch.int32))


@pytest.mark.parametrize("accum,pow2", POLICIES, ids=PID)
@pytest.mark.parametrize("epi", [te.TE_EPI_NONE, te.TE_EPI_DGELU | te.TE_EPI_BGRAD])
@pytest.mark.parametrize("M,N,K", [(384, 384, 512), (256, 128, 256)])
def test_dgrad_quant_transposed(accum, pow2, epi, M, N, K):
    """dZ and dZ^T as e5m2 from one data-gradient call (the bias gradient as the plain call's)."""
    qa, sa = operand(M + 61, M, K, E5, 1e-3, pow2)
    qb, sb = operand(N + 62, N, K, E4, 0.02, pow2)
    zb = W.normal_bf16(np.random.SeedSequence(M + 63), (M, N), 1.28)
    o, d = oracle.gemm_nt(qa, sa, oracle.E5M2, qb, sb, oracle.E4M3)
    has_dg, has_bg = bool(epi & te.TE_EPI_DGELU), bool(epi & te.TE_EPI_BGRAD)
    D, Dm, db, dbm = oracle.dgrad_epilogue(o, d, zb if has_dg else None, has_bg)
    A, SA, B, SB = dev(qa), sdev(sa), dev(qb), sdev(sb)
    Z = bf16_dev(zb) if has_dg else None
    d32h = host(te.te_fp8_gemm_dgrad(A, SA, E5, B, SB, E4, epilogue=epi & ~te.TE_EPI_BGRAD, preact=Z,
                                     dx_dtype=te.TE_DTYPE_F32, accum=accum)).numpy()
    bg = torch.empty((N,), dtype=torch.float32, device="cuda") if has_bg else None
    qt, qts = quant_t_bufs(M, N)
    q, s, _, _ = te.te_fp8_gemm_dgrad_quant(A, SA, E5, B, SB, E4, epilogue=epi, preact=Z, bias_grad=bg,
                                            q_dtype=te.TE_DTYPE_E5M2, accum=accum, transposed=True, qt=qt[:, :M],
                                            qt_scales=qts)
    torch.cuda.synchronize()
    qo, so = oracle.cast_per_token_f32(d32h, oracle.E5M2)
    assert np.array_equal(host(q).numpy(), qo) and np.array_equal(shost(s, M).view(np.uint32), so.view(np.uint32))
    check_quant_t(qt, qts, M, N, d32h, D, Dm, oracle.E5M2, False, chain_gemm(K, epi_chain(epi)), "dgrad qt")
    if has_bg:
        check_f32(host(bg).numpy(), db, dbm, "bias grad (transposed quant)", chain_colsum(K, M, epi_chain(epi)))


def test_fwd_quant_workload():
    """8192 x 14336 x 4096 with bias + GELU, FAST on power-of-two inputs, e4m3 codes for the next
    layer; rows sampled (the cast is per row)."""
    sh = W.FPROP.shapes
    inp = W.fprop_inputs()
    qx, sx = oracle.cast_per_token(inp["x"], oracle.E4M3, True)
    qw, sw = oracle.cast_per_token(inp["w"], oracle.E4M3, True)
    M, N = sh["M"], sh["N"]
    epi = te.TE_EPI_BIAS | te.TE_EPI_GELU
    X, SX, Wd, SW, B = dev(qx), sdev(sx), dev(qw), sdev(sw), bf16_dev(inp["b"])
    y32 = te.te_fp8_gemm_fwd(X, SX, E4, Wd, SW, E4, bias=B, epilogue=epi, y_dtype=te.TE_DTYPE_F32, accum=FAST)
    q, qs, qt, qts = te.te_fp8_gemm_fwd_quant(X, SX, E4, Wd, SW, E4, bias=B, epilogue=epi, accum=FAST,
                                              transposed=True)
    # transposed cast on sampled columns (each is a row of qt: all M tokens of one output feature)
    cols = sample_idx(N, 16, 6)
    yc = host(y32[:, torch.from_numpy(cols).cuda()]).numpy()
    qo, so = oracle.cast_per_token_f32(np.ascontiguousarray(yc.T), oracle.E4M3)
    assert np.array_equal(host(qt).numpy()[cols], qo)
    assert np.array_equal(shost(qts, N)[cols].view(np.uint32), so.view(np.uint32))
    del qt, qts
    rows = sample_idx(M, 24, 5)
    yr = host(y32[torch.from_numpy(rows).cuda()]).numpy()
    qo, so = oracle.cast_per_token_f32(yr, oracle.E4M3)
    qr, sr = host(q).numpy()[rows], shost(qs, M)[rows]
    assert np.array_equal(qr, qo)
    assert np.array_equal(sr.view(np.uint32), so.view(np.uint32))
    # the sampled rows (every column) against the fp64 oracle: the fp32 y and the dequantised codes
    o, d = oracle.gemm_nt(qx[rows], sx[rows], oracle.E4M3, qw, sw, oracle.E4M3)
    y, _, zmag = oracle.fwd_epilogue(o, d, inp["b"], True)
    K = qx.shape[1]
    check_f32(yr, y, zmag * GELU_LIP, "fprop y32 rows", chain_gemm(K, BIAS_CHAIN + GELU_CHAIN))
    check_quant(qr, sr, oracle.E4M3, y, zmag * GELU_LIP, "fprop quant rows vs oracle",
                chain_gemm(K, BIAS_CHAIN + GELU_CHAIN))


def test_fwd_tiny_workload():
    """256x256x512, bias + GELU, fp32 out (and the wgrad out+= call on the same operands)."""
    inp = W.tiny_fprop_inputs()
    qx, sx = oracle.cast_per_token(inp["x"], oracle.E4M3)
    qw, sw = oracle.cast_per_token(inp["w"], oracle.E4M3)
    o, d = oracle.gemm_nt(qx, sx, oracle.E4M3, qw, sw, oracle.E4M3)
    y, z, zmag = oracle.fwd_epilogue(o, d, inp["b"], True)
    for accum in (FULL, FAST):
        yg = te.te_fp8_gemm_fwd(dev(qx), sdev(sx), E4, dev(qw), sdev(sw), E4, bias=bf16_dev(inp["b"]),
                                epilogue=te.TE_EPI_BIAS | te.TE_EPI_GELU, y_dtype=te.TE_DTYPE_F32, accum=accum)
        check_f32(host(yg).numpy(), y, zmag * GELU_LIP, "tiny fwd", chain_gemm(512, BIAS_CHAIN + GELU_CHAIN))
    want, mag = oracle.wgrad(o, d, inp["out0"])
    out = dev(inp["out0"])
    te.te_fp8_wgrad_accum(dev(qx), sdev(sx), E4, dev(qw), sdev(sw), E4, out, FULL)
    check_f32(host(out).numpy(), want, mag, "tiny wgrad", chain_gemm(512, 1))


@pytest.mark.parametrize("accum,pow2", POLICIES, ids=PID)
def test_fwd_workload(accum, pow2):
    sh = W.FPROP.shapes
    inp = W.fprop_inputs()
    qx, sx = oracle.cast_per_token(inp["x"], oracle.E4M3, pow2)
    qw, sw = oracle.cast_per_token(inp["w"], oracle.E4M3, pow2)
    epi = te.TE_EPI_BIAS | te.TE_EPI_GELU | te.TE_EPI_AUX_PREACT
    pre = torch.empty((sh["M"], sh["N"]), dtype=torch.bfloat16, device="cuda")
    yg = te.te_fp8_gemm_fwd(dev(qx), sdev(sx), E4, dev(qw), sdev(sw), E4, bias=bf16_dev(inp["b"]), epilogue=epi,
                            y_dtype=te.TE_DTYPE_BF16, preact=pre, accum=accum)
    rows, cols = sample_idx(sh["M"], 24, 3), sample_idx(sh["N"], 40, 4)
    o, d = grid_entries(qx, sx, oracle.E4M3, qw, sw, oracle.E4M3, rows, cols)
    y, z, zmag = oracle.fwd_epilogue(o, d, inp["b"][cols], True)
    check_bf16(bf16_host_f64(yg)[np.ix_(rows, cols)], y, zmag * GELU_LIP, "fprop y")
    check_bf16(bf16_host_f64(pre)[np.ix_(rows, cols)], z, zmag, "fprop preact")


# ------------------------------------------------------------------ dgrad
DG_EPIS = [te.TE_EPI_NONE, te.TE_EPI_DGELU, te.TE_EPI_BGRAD, te.TE_EPI_DGELU | te.TE_EPI_BGRAD]


@pytest.mark.parametrize("accum,pow2", POLICIES, ids=PID)
@pytest.mark.parametrize("epi", DG_EPIS)
@pytest.mark.parametrize("dxdt", [te.TE_DTYPE_F32, te.TE_DTYPE_BF16])
@pytest.mark.parametrize("M,N,K", [(260, 300, 640), (3, 20, 128)])
def test_dgrad_small(accum, pow2, epi, dxdt, M, N, K, gemm_path):
    qa, sa = operand(M + 21, M, K, E5, 1e-3, pow2)
    qb, sb = operand(N + 22, N, K, E4, 0.02, pow2)
    zb = W.normal_bf16(np.random.SeedSequence(M + 23), (M, N), 1.28)
    o, d = oracle.gemm_nt(qa, sa, oracle.E5M2, qb, sb, oracle.E4M3)
    D, Dm, db, dbm = oracle.dgrad_epilogue(o, d, zb if epi & te.TE_EPI_DGELU else None, bool(epi & te.TE_EPI_BGRAD))
    tdt = torch.float32 if dxdt == te.TE_DTYPE_F32 else torch.bfloat16
    ld = N + 8 - (N + 8) % 8
    dxbuf = torch.full((M, ld), 9.0, dtype=tdt, device="cuda")
    bg = torch.full((N + 4,), 3.0, dtype=torch.float32, device="cuda") if epi & te.TE_EPI_BGRAD else None
    zpad = np.zeros((M, ld), np.uint16)
    zpad[:, :N] = zb
    te.te_fp8_gemm_dgrad(dev(qa), sdev(sa), E5, dev(qb), sdev(sb), E4, epilogue=epi,
                         preact=bf16_dev(zpad)[:, :N] if epi & te.TE_EPI_DGELU else None,
                         bias_grad=bg[:N] if bg is not None else None, dx=dxbuf[:, :N], dx_dtype=dxdt, accum=accum)
    torch.cuda.synchronize()
    xb = host(dxbuf)
    assert torch.all(xb[:, N:] == 9.0), "wrote outside dx"
    if dxdt == te.TE_DTYPE_F32:
        check_f32(xb[:, :N].numpy(), D, Dm, "dgrad dx", chain_gemm(K, epi_chain(epi)))
    else:
        check_bf16(bf16_host_f64(xb[:, :N]), D, Dm, "dgrad dx")
    if bg is not None:
        g = host(bg).numpy()
        assert np.all(g[N:] == 3.0)
        check_f32(g[:N], db, dbm, "bias grad", chain_colsum(K, M, epi_chain(epi)))


@pytest.mark.parametrize("accum,pow2", POLICIES, ids=PID)
@pytest.mark.parametrize("M", [3, 301])
def test_dgrad_bias_grad_ignores_scale_padding(accum, pow2, M, gemm_path):
    """Entries of a scale array past the last row are padding the library never uses.  With M not a
    multiple of 4 the last 16-byte run of every block's row scales holds some; NaN there must leave
    dx, its quantised cast and the deterministic bias gradient bit-identical to the calls whose
    padding is zero, and the atomic bias gradients (whose order of additions varies) within the
    bound of the oracle."""
    N, K = 384, 256
    qa, sa = operand(M + 71, M, K, E5, 1e-3, pow2)
    qb, sb = operand(N + 72, N, K, E4, 0.02, pow2)
    zb = W.normal_bf16(np.random.SeedSequence(M + 73), (M, N), 1.28)
    A, B, SB, Z = dev(qa), dev(qb), sdev(sb), bf16_dev(zb)
    DB = te.TE_EPI_DGELU | te.TE_EPI_BGRAD
    runs = {}
    for fill in (0.0, float("nan")):
        SA = sdev(sa, fill)
        bg = torch.empty((N,), dtype=torch.float32, device="cuda")
        dx = te.te_fp8_gemm_dgrad(A, SA, E5, B, SB, E4, epilogue=DB, preact=Z, bias_grad=bg, accum=accum)
        bgd = torch.empty((N,), dtype=torch.float32, device="cuda")
        te.te_fp8_gemm_dgrad_deterministic(A, SA, E5, B, SB, E4, bgd, epilogue=DB, preact=Z, accum=accum)
        bgq = torch.empty((N,), dtype=torch.float32, device="cuda")
        q, qs = te.te_fp8_gemm_dgrad_quant(A, SA, E5, B, SB, E4, epilogue=DB, preact=Z, bias_grad=bgq,
                                           accum=accum)
        torch.cuda.synchronize()
        runs[fill == 0.0] = [host(t) for t in (dx, bg, bgd, bgq, q)] + [host(qs)[:, :M].contiguous()]
    for k, what in ((0, "dx"), (2, "deterministic bias grad"), (4, "q"), (5, "q scales")):
        a, b = runs[True][k], runs[False][k]
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{what}: the scale padding changed the result"
    o, d = oracle.gemm_nt(qa, sa, oracle.E5M2, qb, sb, oracle.E4M3)
    _, _, db, dbm = oracle.dgrad_epilogue(o, d, zb, True)
    for k in (1, 2, 3):
        check_f32(runs[False][k].numpy(), db, dbm, "bias grad (NaN scale padding)", chain_colsum(K, M, epi_chain(DB)))


DGRAD_EPIS = [te.TE_EPI_NONE, te.TE_EPI_DGELU, te.TE_EPI_DGELU | te.TE_EPI_BGRAD]


@pytest.mark.parametrize("accum,pow2", POLICIES, ids=PID)
@pytest.mark.parametrize("epi", DGRAD_EPIS)
@pytest.mark.parametrize("qdt,cast_pow2", [(te.TE_DTYPE_E5M2, False), (te.TE_DTYPE_E4M3, False),
                                           (te.TE_DTYPE_E5M2, True)])
@pytest.mark.parametrize("M,N,K", [(300, 384, 512), (40, 128, 256)])
def test_dgrad_quant(accum, pow2, epi, qdt, cast_pow2, M, N, K, gemm_path):
    """The quantised dgrad equals the per-token cast of the dgrad's own fp32 D (the oracle's
    fp32-input cast of the fp32 dx the plain call returns), that fp32 D and the bias gradient match
    the fp64 oracle, and nothing outside q, its scales and the bias gradient is written."""
    qa, sa = operand(M + 31, M, K, E5, 1e-3, pow2)
    qb, sb = operand(N + 32, N, K, E4, 0.02, pow2)
    zb = W.normal_bf16(np.random.SeedSequence(M + 33), (M, N), 1.28)
    o, d = oracle.gemm_nt(qa, sa, oracle.E5M2, qb, sb, oracle.E4M3)
    has_dg, has_bg = bool(epi & te.TE_EPI_DGELU), bool(epi & te.TE_EPI_BGRAD)
    D, Dm, db, dbm = oracle.dgrad_epilogue(o, d, zb if has_dg else None, has_bg)
    A, SA, B, SB = dev(qa), sdev(sa), dev(qb), sdev(sb)
    Z = bf16_dev(zb) if has_dg else None
    d32 = te.te_fp8_gemm_dgrad(A, SA, E5, B, SB, E4, epilogue=epi & ~te.TE_EPI_BGRAD, preact=Z,
                               dx_dtype=te.TE_DTYPE_F32, accum=accum)
    d32h = host(d32).numpy()
    check_f32(d32h, D, Dm, "dgrad D (fp32)", chain_gemm(K, epi_chain(epi)))
    qbuf = torch.full((M, N + 16), 0xA5, dtype=torch.uint8, device="cuda")
    qs = torch.full((N // 128, scale_ld(M)), -3.0, dtype=torch.float32, device="cuda")
    bg = torch.full((N + 4,), 3.0, dtype=torch.float32, device="cuda") if has_bg else None
    te.te_fp8_gemm_dgrad_quant(A, SA, E5, B, SB, E4, epilogue=epi, preact=Z, bias_grad=bg[:N] if has_bg else None,
                               q_dtype=qdt, cast_flags=te.TE_CAST_POW2_SCALE if cast_pow2 else 0, q=qbuf[:, :N],
                               q_scales=qs, accum=accum)
    torch.cuda.synchronize()
    qh, sh = host(qbuf).numpy(), host(qs).numpy()
    assert (qh[:, N:] == 0xA5).all() and (sh[:, M:] == -3.0).all()
    qo, so = oracle.cast_per_token_f32(d32h, OF[qdt], cast_pow2)
    bad = np.argwhere(qh[:, :N] != qo)
    assert bad.size == 0, f"{len(bad)} code mismatches, first {bad[0]}"
    assert np.array_equal(shost(qs, M).view(np.uint32), so.view(np.uint32)), "scale mismatch"
    check_quant(qh[:, :N], shost(qs, M), OF[qdt], D, Dm, "dgrad quant vs oracle", chain_gemm(K, epi_chain(epi)))
    if has_bg:
        g = host(bg).numpy()
        assert np.all(g[N:] == 3.0)
        check_f32(g[:N], db, dbm, "bias grad", chain_colsum(K, M, epi_chain(epi)))


@pytest.mark.parametrize("accum,pow2", POLICIES, ids=PID)
@pytest.mark.parametrize("epi", [te.TE_EPI_BGRAD, te.TE_EPI_DGELU | te.TE_EPI_BGRAD])
@pytest.mark.parametrize("M,N,K", [(300, 264, 512), (600, 37, 128)])
def test_dgrad_deterministic_bias_grad(accum, pow2, epi, M, N, K, gemm_path):
    """The atomic-free bias gradient: within tolerance of the oracle, bit-identical from run to run,
    and the dx it writes is the plain call's dx bit for bit."""
    qa, sa = operand(M + 41, M, K, E5, 1e-3, pow2)
    qb, sb = operand(N + 42, N, K, E4, 0.02, pow2)
    zb = W.normal_bf16(np.random.SeedSequence(M + 43), (M, N), 1.28)
    o, d = oracle.gemm_nt(qa, sa, oracle.E5M2, qb, sb, oracle.E4M3)
    has_dg = bool(epi & te.TE_EPI_DGELU)
    _, _, db, dbm = oracle.dgrad_epilogue(o, d, zb if has_dg else None, True)
    A, SA, B, SB = dev(qa), sdev(sa), dev(qb), sdev(sb)
    zpad = np.zeros((M, N + 8 - N % 8), np.uint16)
    zpad[:, :N] = zb
    Z = bf16_dev(zpad)[:, :N] if has_dg else None
    ld = N + 4 - N % 4
    runs = []
    for _ in range(3):
        bg = torch.full((N,), 7.0, dtype=torch.float32, device="cuda")
        ws = torch.full((te.load_library().te_fp8_dgrad_bgrad_workspace_bytes(M, N) // 4,), float("nan"),
                        dtype=torch.float32, device="cuda")
        dx = torch.empty((M, ld), dtype=torch.float32, device="cuda")[:, :N]
        te.te_fp8_gemm_dgrad_deterministic(A, SA, E5, B, SB, E4, bg, epilogue=epi, preact=Z, workspace=ws, dx=dx,
                                           dx_dtype=te.TE_DTYPE_F32, accum=accum)
        runs.append((host(bg).numpy(), host(dx).numpy()))
    for g, _ in runs[1:]:
        assert np.array_equal(g.view(np.uint32), runs[0][0].view(np.uint32)), "bias grad not deterministic"
    check_f32(runs[0][0], db, dbm, "deterministic bias grad", chain_colsum(K, M, epi_chain(epi)))
    ref = torch.empty((M, ld), dtype=torch.float32, device="cuda")[:, :N]
    te.te_fp8_gemm_dgrad(A, SA, E5, B, SB, E4, epilogue=epi & ~te.TE_EPI_BGRAD, preact=Z, dx=ref,
                         dx_dtype=te.TE_DTYPE_F32, accum=accum)
    assert np.array_equal(runs[0][1].view(np.uint32), host(ref).numpy().view(np.uint32))


@pytest.mark.parametrize("accum", [FULL, FAST])
def test_dgrad_workload_dx(accum):
    """dX[8192x4096] = dY[8192x14336] (e5m2) W^T (e4m3), bf16 out."""
    sh = W.DGRAD.shapes
    inp = W.dgrad_inputs()
    qa, sa = oracle.cast_per_token(inp["dy"], oracle.E5M2)
    qb, sb = oracle.cast_per_token(inp["wt"], oracle.E4M3)
    dx = te.te_fp8_gemm_dgrad(dev(qa), sdev(sa), E5, dev(qb), sdev(sb), E4, accum=accum)
    rows, cols = sample_idx(sh["M"], 24, 5), sample_idx(sh["N"], 40, 6)
    o, d = grid_entries(qa, sa, oracle.E5M2, qb, sb, oracle.E4M3, rows, cols)
    check_bf16(bf16_host_f64(dx)[np.ix_(rows, cols)], o, d, "dgrad dX")


@pytest.mark.parametrize("accum", [FULL, FAST])
def test_dgrad_workload_dgelu_bgrad(accum):
    """dZ[8192x14336] = dO (e5m2) W2^T (e4m3) through GELU'(Z), bias grad = its column sums.  dZ in
    fp32 on a sampled grid against the oracle; the bias gradient on every column against the fp64
    column sums of that same fp32 dZ, and on sampled columns against the oracle; the bf16 store is
    the round-to-nearest-even of the fp32 one."""
    sh = W.DGRAD.shapes
    M, N, K = sh["M"], sh["K"], sh["N"]  # the pre-activation GEMM: out features 14336, contraction 4096
    inp = W.dgrad_inputs()
    qa, sa = oracle.cast_per_token(inp["do"], oracle.E5M2)
    qb, sb = oracle.cast_per_token(inp["w2t"], oracle.E4M3)
    z = inp["z"]
    A, SA, B, SB, Z = dev(qa), sdev(sa), dev(qb), sdev(sb), bf16_dev(z)
    epi = te.TE_EPI_DGELU | te.TE_EPI_BGRAD
    bg = torch.empty((N,), dtype=torch.float32, device="cuda")
    dz = te.te_fp8_gemm_dgrad(A, SA, E5, B, SB, E4, epilogue=epi, preact=Z, bias_grad=bg,
                              dx_dtype=te.TE_DTYPE_F32, accum=accum)
    rows, cols = sample_idx(M, 16, 7), sample_idx(N, 24, 8)
    o, d = grid_entries(qa, sa, oracle.E5M2, qb, sb, oracle.E4M3, rows, cols)
    D, Dm, _, _ = oracle.dgrad_epilogue(o, d, z[np.ix_(rows, cols)])
    dzh = host(dz).numpy()
    check_f32(dzh[np.ix_(rows, cols)], D, Dm, "dZ fp32", chain_gemm(K, GELU_CHAIN))
    g = host(bg).numpy()
    # every column: the kernel's own fp32 dZ summed in fp64
    cs = dzh.astype(np.float64).sum(0)
    csm = np.abs(dzh.astype(np.float64)).sum(0)
    check_f32(g, cs, csm, "bias grad vs colsum(dZ)", 4 + 4 + (M + 63) // 64, mma=False)
    bcols = cols[:8]
    o, d = grid_entries(qa, sa, oracle.E5M2, qb, sb, oracle.E4M3, np.arange(M), bcols)
    _, _, db, dbm = oracle.dgrad_epilogue(o, d, z[:, bcols], bgrad=True)
    check_f32(g[bcols], db, dbm, "bias grad", chain_colsum(K, M, GELU_CHAIN))
    del dz
    if accum == FULL:
        dzb = te.te_fp8_gemm_dgrad(A, SA, E5, B, SB, E4, epilogue=epi, preact=Z, bias_grad=bg, accum=accum)
        assert torch.equal(host(dzb).view(torch.int16), torch.from_numpy(dzh).to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("M,N,K", [(300, 264, 384), (512, 768, 1024)])
def test_fast_on_ieee_scales_is_full_bit_for_bit(M, N, K, gemm_path):
    """TE_ACCUM_FAST chains through the matrix core only where a tile's scales are powers of two;
    on IEEE-scaled operands (the default cast) every tile takes the FULL promotion, so each entry
    point's FAST result is its FULL result bit for bit (the reason the training modules ask for FULL
    when their casts use IEEE scales)."""
    qa, sa = operand(151, M, K, E4)
    qb, sb = operand(152, N, K, E4, 0.05)
    qd, sd = operand(153, M, K, E5, 1e-3)
    A, SA, B, SB, D, SD = dev(qa), sdev(sa), dev(qb), sdev(sb), dev(qd), sdev(sd)
    b = bf16_dev(W.normal_bf16(np.random.SeedSequence(154), (N,), 0.1))
    Z = bf16_dev(W.normal_bf16(np.random.SeedSequence(155), (M, N), 1.28))
    out0 = dev(W.normal_f32(np.random.SeedSequence(156), (M, N)))
    res = {}
    for accum in (FULL, FAST):
        y = te.te_fp8_gemm_fwd(A, SA, E4, B, SB, E4, bias=b, epilogue=te.TE_EPI_BIAS | te.TE_EPI_GELU,
                               y_dtype=te.TE_DTYPE_F32, accum=accum)
        bg = torch.empty((N,), dtype=torch.float32, device="cuda")
        dz = te.te_fp8_gemm_dgrad_deterministic(D, SD, E5, B, SB, E4, bg, epilogue=te.TE_EPI_DGELU | te.TE_EPI_BGRAD,
                                                preact=Z, dx_dtype=te.TE_DTYPE_F32, accum=accum)
        out = out0.clone()
        te.te_fp8_wgrad_accum(A, SA, E4, B, SB, E4, out, accum)
        res[accum] = [host(t) for t in (y, dz, bg, out)]
    for what, f, g in zip(("fwd", "dgrad", "bias grad", "wgrad"), res[FULL], res[FAST]):
        assert torch.equal(f.view(torch.int32), g.view(torch.int32)), f"{what}: FAST on IEEE scales differs from FULL"


def spread_operand(seed, rows, K, dt, pow2):
    """An operand whose rows span 2^-12 .. 2^12 in magnitude, so its per-row scales (and their
    E8M0 exponents, where they are powers of two) differ widely."""
    rng = np.random.default_rng(seed)
    mag = np.exp2(rng.integers(-12, 13, (rows, 1))).astype(np.float32)
    bits = W.f32_to_bf16_bits(rng.standard_normal((rows, K), dtype=np.float32) * mag)
    return oracle.cast_per_token(bits, OF[dt], pow2)


@pytest.mark.parametrize("M,N,K", [(300, 264, 384), (512, 768, 1024)])
def test_fast_on_one_pow2_operand_is_full_bit_for_bit(M, N, K, gemm_path):
    """Power-of-two scales on one operand only (B: the backward products of a pow2_scales module,
    IEEE-scaled gradients times power-of-two-scaled forward operands; or A): the matrix core may
    chain only where both operands' scales are powers of two, so every tile takes the FULL
    promotion and each entry point's FAST result is its FULL result bit for bit.  The operands'
    rows span 2^-12 .. 2^12, so a scale wrongly taken as an E8M0 exponent would show."""
    qa, sa = spread_operand(161, M, K, E5, False)
    qb, sb = spread_operand(162, N, K, E4, True)
    qp, sp = spread_operand(163, M, K, E5, True)
    qi, si = spread_operand(164, N, K, E4, False)
    b = bf16_dev(W.normal_bf16(np.random.SeedSequence(165), (N,), 0.1))
    Z = bf16_dev(W.normal_bf16(np.random.SeedSequence(166), (M, N), 1.28))
    out0 = dev(W.normal_f32(np.random.SeedSequence(167), (M, N)))
    for what, (A, SA, B, SB) in (("pow2 B", (dev(qa), sdev(sa), dev(qb), sdev(sb))),
                                 ("pow2 A", (dev(qp), sdev(sp), dev(qi), sdev(si)))):
        res = {}
        for accum in (FULL, FAST):
            y = te.te_fp8_gemm_fwd(A, SA, E5, B, SB, E4, bias=b, epilogue=te.TE_EPI_BIAS | te.TE_EPI_GELU,
                                   y_dtype=te.TE_DTYPE_F32, accum=accum)
            bg = torch.empty((N,), dtype=torch.float32, device="cuda")
            dz = te.te_fp8_gemm_dgrad_deterministic(A, SA, E5, B, SB, E4, bg,
                                                    epilogue=te.TE_EPI_DGELU | te.TE_EPI_BGRAD, preact=Z,
                                                    dx_dtype=te.TE_DTYPE_F32, accum=accum)
            out = out0.clone()
            te.te_fp8_wgrad_accum(A, SA, E5, B, SB, E4, out, accum)
            res[accum] = [host(t) for t in (y, dz, bg, out)]
        for op, f, g in zip(("fwd", "dgrad", "bias grad", "wgrad"), res[FULL], res[FAST]):
            assert torch.equal(f.view(torch.int32), g.view(torch.int32)), f"{what}, {op}: FAST differs from FULL"
    # and the FAST result against the oracle
    o, d = oracle.gemm_nt(qa, sa, OF[E5], qb, sb, OF[E4])
    want, mag = oracle.wgrad(o, d, host(out0).numpy())
    out = out0.clone()
    te.te_fp8_wgrad_accum(dev(qa), sdev(sa), E5, dev(qb), sdev(sb), E4, out, FAST)
    check_f32(host(out).numpy(), want, mag, "wgrad, pow2 B only, on FAST", chain_gemm(K, 1))


# ------------------------------------------------------------------ M-grouped
def mgrouped_case(seed, G, blocks, N, K, pow2=False, fx=E4, wstd=0.05):
    sum_m = 256 * len(blocks)
    qx, sx = operand(seed, sum_m, K, fx, pow2=pow2)
    ws = [operand(seed + 1 + e, N, K, E4, std=wstd, pow2=pow2) for e in range(G)]
    qw = np.stack([w[0] for w in ws])
    sw = np.stack([w[1] for w in ws])
    b = W.normal_bf16(np.random.SeedSequence(seed + 100), (G, N), 0.1)
    return qx, sx, qw, sw, b


def w_dev(qw, sw):
    """Expert operands and scales in the layout the M-grouped call takes."""
    return dev(qw), torch.stack([sdev(sw[e]) for e in range(sw.shape[0])]).contiguous()


@pytest.mark.parametrize("accum,pow2", POLICIES, ids=PID)
@pytest.mark.parametrize("epi,ydt", [(te.TE_EPI_NONE, te.TE_DTYPE_F32),
                                     (te.TE_EPI_BIAS | te.TE_EPI_GELU, te.TE_DTYPE_F32),
                                     (te.TE_EPI_BIAS | te.TE_EPI_GELU | te.TE_EPI_AUX_PREACT, te.TE_DTYPE_BF16)])
def test_mgrouped_fwd(accum, pow2, epi, ydt, gemm_path):
    """Blocks of 256 token rows, each with its expert (or -1: skipped, rows untouched); N ragged."""
    blocks = np.array([2, 0, -1, 2, 1], np.int32)
    G, N, K = 3, 200, 384
    qx, sx, qw, sw, b = mgrouped_case(70, G, blocks, N, K, pow2)
    y, z, zmag = oracle.mgrouped_fwd(qx, sx, oracle.E4M3, qw, sw, oracle.E4M3, blocks,
                                     b if epi & te.TE_EPI_BIAS else None, bool(epi & te.TE_EPI_GELU))
    tdt = torch.float32 if ydt == te.TE_DTYPE_F32 else torch.bfloat16
    M = 256 * len(blocks)
    ybuf = torch.full((M, N + 8), 77.0, dtype=tdt, device="cuda")
    pre = None
    if epi & te.TE_EPI_AUX_PREACT:
        prebuf = torch.full((M, N + 8), 55.0, dtype=torch.bfloat16, device="cuda")
        pre = prebuf[:, :N]
    wq, ws = w_dev(qw, sw)
    te.te_fp8_mgrouped_gemm_fwd(dev(qx), sdev(sx), E4, wq, ws, E4, torch.from_numpy(blocks).cuda(),
                                bias=bf16_dev(b) if epi & te.TE_EPI_BIAS else None, epilogue=epi,
                                y=ybuf[:, :N], y_dtype=ydt, preact=pre, accum=accum)
    torch.cuda.synchronize()
    yb = host(ybuf)
    assert torch.all(yb[:, N:] == 77.0), "wrote past N"
    live = np.repeat(blocks >= 0, 256)
    assert torch.all(yb[torch.from_numpy(~live)] == 77.0), "a skipped block was written"
    ymag = zmag * (GELU_LIP if epi & te.TE_EPI_GELU else 1.0)
    if ydt == te.TE_DTYPE_F32:
        check_f32(yb[:, :N].numpy()[live], y[live], ymag[live], "mgrouped y", chain_gemm(K, epi_chain(epi)))
    else:
        check_bf16(bf16_host_f64(yb[:, :N])[live], y[live], ymag[live], "mgrouped y")
    if pre is not None:
        pb = host(prebuf)
        assert torch.all(pb[torch.from_numpy(~live)] == 55.0)
        check_bf16(bf16_host_f64(pb[:, :N])[live], z[live], zmag[live], "mgrouped preact")


def test_mgrouped_dgrad_form_e5m2():
    """The data gradient of an expert layer: dY (e5m2) blocks times each expert's W^T, no epilogue, bf16."""
    blocks = np.array([1, 1, 0, 3, -1, 2], np.int32)
    G, N, K = 4, 512, 640
    qx, sx, qw, sw, _ = mgrouped_case(80, G, blocks, N, K, fx=te.TE_DTYPE_E5M2)
    y, _, zmag = oracle.mgrouped_fwd(qx, sx, oracle.E5M2, qw, sw, oracle.E4M3, blocks)
    wq, ws = w_dev(qw, sw)
    yg = te.te_fp8_mgrouped_gemm_fwd(dev(qx), sdev(sx), te.TE_DTYPE_E5M2, wq, ws, E4,
                                     torch.from_numpy(blocks).cuda(), y_dtype=te.TE_DTYPE_BF16, accum=FULL)
    live = np.repeat(blocks >= 0, 256)
    # (rows of a skipped block are never written: the buffer's own contents, not converted)
    check_bf16(bf16_host_f64(yg[torch.from_numpy(live).cuda()]), y[live], zmag[live], "mgrouped dX")


@pytest.mark.parametrize("accum,pow2", POLICIES, ids=PID)
@pytest.mark.parametrize("epi,dxdt", [(te.TE_EPI_DGELU | te.TE_EPI_BGRAD, te.TE_DTYPE_F32),
                                      (te.TE_EPI_BGRAD, te.TE_DTYPE_BF16), (te.TE_EPI_DGELU, te.TE_DTYPE_BF16)])
def test_mgrouped_dgrad(accum, pow2, epi, dxdt, gemm_path):
    """Per-expert data gradient through GELU' with per-expert bias gradients: each live block is
    the dense dgrad epilogue with its expert's W^T; bias_grad[e] sums expert e's blocks (an expert
    with no block gets zeros); skipped blocks are not written."""
    blocks = np.array([1, 0, -1, 1, 2], np.int32)
    G, N, K = 4, 200, 384
    M = 256 * len(blocks)
    qa, sa = operand(110, M, K, E5, 1e-3, pow2)
    ws = [operand(111 + e, N, K, E4, 0.02, pow2) for e in range(G)]
    qw, sw = np.stack([w[0] for w in ws]), np.stack([w[1] for w in ws])
    zb = W.normal_bf16(np.random.SeedSequence(120), (M, N), 1.28)
    has_dg, has_bg = bool(epi & te.TE_EPI_DGELU), bool(epi & te.TE_EPI_BGRAD)
    D, Dm, db, dbm = oracle.mgrouped_dgrad(qa, sa, oracle.E5M2, qw, sw, oracle.E4M3, blocks, zb if has_dg else None)
    tdt = torch.float32 if dxdt == te.TE_DTYPE_F32 else torch.bfloat16
    dxbuf = torch.full((M, N + 8), 9.0, dtype=tdt, device="cuda")
    bg = torch.full((G * N,), 3.0, dtype=torch.float32, device="cuda") if has_bg else None
    zpad = np.zeros((M, N + 8), np.uint16)
    zpad[:, :N] = zb
    wq, wsd = w_dev(qw, sw)
    te.te_fp8_mgrouped_gemm_dgrad(dev(qa), sdev(sa), E5, wq, wsd, E4, torch.from_numpy(blocks).cuda(), epilogue=epi,
                                  preact=bf16_dev(zpad)[:, :N] if has_dg else None, bias_grad=bg, dx=dxbuf[:, :N],
                                  dx_dtype=dxdt, accum=accum)
    torch.cuda.synchronize()
    xb = host(dxbuf)
    live = np.repeat(blocks >= 0, 256)
    assert torch.all(xb[:, N:] == 9.0) and torch.all(xb[torch.from_numpy(~live)] == 9.0)
    if dxdt == te.TE_DTYPE_F32:
        check_f32(xb[:, :N].numpy()[live], D[live], Dm[live], "mgrouped dgrad D", chain_gemm(K, epi_chain(epi)))
    else:
        check_bf16(bf16_host_f64(xb[:, :N])[live], D[live], Dm[live], "mgrouped dgrad D")
    if has_bg:
        g = host(bg).numpy().reshape(G, N)
        assert (g[3] == 0).all(), "an expert without blocks must get a zero bias gradient"
        check_f32(g[:3], db[:3], dbm[:3], "per-expert bias grad", chain_colsum(K, M, epi_chain(epi)))


@pytest.mark.parametrize("accum,pow2", POLICIES, ids=PID)
@pytest.mark.parametrize("epi", [te.TE_EPI_BGRAD, te.TE_EPI_DGELU | te.TE_EPI_BGRAD])
def test_mgrouped_dgrad_deterministic(accum, pow2, epi, gemm_path):
    """The atomic-free per-expert bias gradient: within the oracle bound, bit-identical from run to
    run (with the workspace refilled with garbage in between), an expert with no block gets zeros,
    and dx is the atomic call's dx bit for bit."""
    blocks = np.array([2, 0, -1, 2, 0, 5], np.int32)     # expert 1 has no block; -1 and 5 (>= G) are skipped
    G, N, K = 4, 200, 256
    M = 256 * len(blocks)
    qa, sa = operand(130, M, K, E5, 1e-3, pow2)
    ws = [operand(131 + e, N, K, E4, 0.02, pow2) for e in range(G)]
    qw, sw = np.stack([w[0] for w in ws]), np.stack([w[1] for w in ws])
    zb = W.normal_bf16(np.random.SeedSequence(140), (M, N), 1.28)
    has_dg = bool(epi & te.TE_EPI_DGELU)
    D, Dm, db, dbm = oracle.mgrouped_dgrad(qa, sa, oracle.E5M2, qw, sw, oracle.E4M3, blocks, zb if has_dg else None)
    zpad = np.zeros((M, N + 8), np.uint16)
    zpad[:, :N] = zb
    Z = bf16_dev(zpad)[:, :N] if has_dg else None
    A, SA = dev(qa), sdev(sa)
    wq, wsd = w_dev(qw, sw)
    mb = torch.from_numpy(blocks).cuda()
    work = torch.empty((te.load_library().te_fp8_dgrad_bgrad_workspace_bytes(M, N),), dtype=torch.uint8,
                       device="cuda")
    runs = []
    for r in range(2):
        work.fill_(0xFF if r else 0x7F)          # NaN / large garbage: unwritten rows must not be read
        bg = torch.full((G * N,), 3.0, dtype=torch.float32, device="cuda")
        dx = te.te_fp8_mgrouped_gemm_dgrad_deterministic(A, SA, E5, wq, wsd, E4, mb, bg, epilogue=epi, preact=Z,
                                                         workspace=work, accum=accum)
        torch.cuda.synchronize()
        runs.append((host(bg), host(dx)))
    assert torch.equal(runs[0][0].view(torch.int32), runs[1][0].view(torch.int32)), "bias gradient not reproducible"
    g = runs[0][0].numpy().reshape(G, N)
    assert (g[1] == 0).all() and (g[3] == 0).all(), "an expert without blocks must get a zero bias gradient"
    check_f32(g[[0, 2]], db[[0, 2]], dbm[[0, 2]], "per-expert bias grad (deterministic)",
              chain_colsum(K, M, epi_chain(epi)))
    bga = torch.empty((G * N,), dtype=torch.float32, device="cuda")
    dxa = te.te_fp8_mgrouped_gemm_dgrad(A, SA, E5, wq, wsd, E4, mb, epilogue=epi, preact=Z, bias_grad=bga,
                                        accum=accum)
    live = torch.from_numpy(np.repeat((blocks >= 0) & (blocks < G), 256))
    assert torch.equal(host(dxa)[live].view(torch.int16), runs[0][1][live].view(torch.int16))


def test_mgrouped_same_expert_equals_dense(gemm_path):
    """With every block on one expert the call is the dense forward GEMM, bit for bit."""
    blocks = np.zeros(4, np.int32)
    qx, sx, qw, sw, b = mgrouped_case(90, 1, blocks, 384, 512)
    epi = te.TE_EPI_BIAS | te.TE_EPI_GELU
    wq, ws = w_dev(qw, sw)
    yg = te.te_fp8_mgrouped_gemm_fwd(dev(qx), sdev(sx), E4, wq, ws, E4, torch.from_numpy(blocks).cuda(),
                                     bias=bf16_dev(b), epilogue=epi, y_dtype=te.TE_DTYPE_F32, accum=FULL)
    yd = te.te_fp8_gemm_fwd(dev(qx), sdev(sx), E4, dev(qw[0]), sdev(sw[0]), E4, bias=bf16_dev(b[0]), epilogue=epi,
                            y_dtype=te.TE_DTYPE_F32, accum=FULL)
    assert torch.equal(host(yg).view(torch.int32), host(yd).view(torch.int32))


# ------------------------------------------------------------------ K-grouped
@pytest.mark.parametrize("accum,pow2", POLICIES, ids=PID)
def test_kgrouped_small(accum, pow2, gemm_path):
    gk = np.array([256, 0, 128, 384, 0, 128], np.int64)
    M, N, S = 200, 300, int(gk.sum())
    qa, sa = operand(31, M, S, E4, pow2=pow2)
    qb, sb = operand(32, N, S, E4, pow2=pow2)
    init = W.normal_f32(np.random.SeedSequence(33), (len(gk), M, N))
    want, mag = oracle.kgrouped_wgrad(qa, sa, oracle.E4M3, qb, sb, oracle.E4M3, gk, init)
    out = dev(init)
    te.te_fp8_kgrouped_wgrad(dev(qa), sdev(sa), E4, dev(qb), sdev(sb), E4, gk.tolist(), out, accum)
    got = host(out).numpy()
    for g in range(len(gk)):
        if gk[g] == 0:
            assert np.array_equal(got[g].view(np.uint32), init[g].view(np.uint32)), f"empty group {g} touched"
        else:
            check_f32(got[g], want[g], mag[g], f"group {g}", chain_gemm(gk[g], 1))


def test_kgrouped_many_groups(gemm_path):
    """More groups than one launch carries: 300 groups of 128 or 0 columns."""
    rng = np.random.default_rng(4)
    gk = (rng.integers(0, 2, 300) * 128).astype(np.int64)
    gk[0] = 128
    M, N, S = 16, 24, int(gk.sum())
    qa, sa = operand(41, M, S, E4)
    qb, sb = operand(42, N, S, E4)
    init = W.normal_f32(np.random.SeedSequence(43), (len(gk), M, N))
    want, mag = oracle.kgrouped_wgrad(qa, sa, oracle.E4M3, qb, sb, oracle.E4M3, gk, init)
    out = dev(init)
    te.te_fp8_kgrouped_wgrad(dev(qa), sdev(sa), E4, dev(qb), sdev(sb), E4, gk.tolist(), out, FULL)
    check_f32(host(out).numpy(), want, mag, "300 groups", chain_gemm(128, 1))


@pytest.mark.parametrize("accum,pow2", POLICIES, ids=PID)
def test_kgrouped_device_sizes_matches_host_sizes(accum, pow2, gemm_path):
    """Group sizes read from device memory: bit-identical to the host-sized call (the tiles do the
    same arithmetic; only their order differs), within tolerance of the oracle, empty groups untouched
    (including the sign of zero), and columns past the groups' sum unused."""
    gk = np.array([256, 0, 128, 384, 0, 128], np.int64)
    M, N, S = 200, 300, int(gk.sum()) + 256          # 256 trailing columns belong to no group
    qa, sa = operand(51, M, S, E4, pow2=pow2)
    qb, sb = operand(52, N, S, E4, pow2=pow2)
    init = W.normal_f32(np.random.SeedSequence(53), (len(gk), M, N))
    init[1, :7, :5] = -0.0
    cut = int(gk.sum())
    qa_c, sa_c = np.ascontiguousarray(qa[:, :cut]), np.ascontiguousarray(sa[:, :cut // 128])
    qb_c, sb_c = np.ascontiguousarray(qb[:, :cut]), np.ascontiguousarray(sb[:, :cut // 128])
    want, mag = oracle.kgrouped_wgrad(qa_c, sa_c, oracle.E4M3, qb_c, sb_c, oracle.E4M3, gk, init)
    out_d = dev(init)
    te.te_fp8_kgrouped_wgrad_device_sizes(dev(qa), sdev(sa), E4, dev(qb), sdev(sb), E4,
                                          torch.from_numpy(gk).cuda(), out_d, accum)
    got = host(out_d).numpy()
    # the host-sized call on the operands cut to the groups' columns
    out_h = dev(init)
    te.te_fp8_kgrouped_wgrad(dev(qa_c), sdev(sa_c), E4, dev(qb_c), sdev(sb_c), E4, gk.tolist(), out_h, accum)
    assert np.array_equal(got.view(np.uint32), host(out_h).numpy().view(np.uint32))
    for g in range(len(gk)):
        if gk[g] == 0:
            assert np.array_equal(got[g].view(np.uint32), init[g].view(np.uint32)), f"empty group {g} touched"
        else:
            check_f32(got[g], want[g], mag[g], f"group {g}", chain_gemm(gk[g], 1))


def test_kgrouped_device_sizes_follow_the_device_array():
    """The sizes are read when the kernel runs: changing them on the device (no host copy) between two
    calls changes which columns each group takes."""
    M, N, S = 64, 96, 1024
    qa, sa = operand(61, M, S, E4)
    qb, sb = operand(62, N, S, E4)
    A, SA, B, SB = dev(qa), sdev(sa), dev(qb), sdev(sb)
    first, second = np.array([512, 512], np.int64), np.array([128, 768], np.int64)
    gk = torch.from_numpy(first).cuda()
    init = W.normal_f32(np.random.SeedSequence(63), (2, M, N))
    out = dev(init)
    te.te_fp8_kgrouped_wgrad_device_sizes(A, SA, E4, B, SB, E4, gk, out, FULL)
    gk.copy_(torch.from_numpy(second).cuda())        # device-to-device update, stream-ordered
    te.te_fp8_kgrouped_wgrad_device_sizes(A, SA, E4, B, SB, E4, gk, out, FULL)
    o1, d1 = oracle.kgrouped_wgrad(qa, sa, oracle.E4M3, qb, sb, oracle.E4M3, first, init)
    want, mag = oracle.kgrouped_wgrad(np.ascontiguousarray(qa[:, :896]), np.ascontiguousarray(sa[:, :7]), oracle.E4M3,
                                      np.ascontiguousarray(qb[:, :896]), np.ascontiguousarray(sb[:, :7]), oracle.E4M3,
                                      second, o1)
    check_f32(host(out).numpy(), want, mag + d1, "two calls", chain_gemm(S, 2))


def test_kgrouped_device_sizes_workload():
    """The 8-expert workload with its multinomial token counts on the device."""
    sh = W.KGROUPED.shapes
    inp = W.kgrouped_inputs()
    gk = inp["group_k"]
    qa, sa = oracle.cast_per_token(inp["a"], oracle.E4M3)
    qb, sb = oracle.cast_per_token(inp["b"], oracle.E4M3)
    out = dev(inp["out0"])
    te.te_fp8_kgrouped_wgrad_device_sizes(dev(qa), sdev(sa), E4, dev(qb), sdev(sb), E4,
                                          torch.from_numpy(np.asarray(gk, np.int64)).cuda(), out, FULL)
    got = host(out).numpy()
    offs = np.concatenate([[0], np.cumsum(gk)])
    for g in range(sh["G"]):
        rows, cols = sample_idx(sh["M"], 8, 30 + g), sample_idx(sh["N"], 12, 40 + g)
        o, d = grid_entries(qa, sa, oracle.E4M3, qb, sb, oracle.E4M3, rows, cols, int(offs[g]), int(gk[g]))
        want, mag = oracle.wgrad(o, d, inp["out0"][g][np.ix_(rows, cols)])
        check_f32(got[g][np.ix_(rows, cols)], want, mag, f"expert {g}", chain_gemm(gk[g], 1))


def test_kgrouped_workload():
    sh = W.KGROUPED.shapes
    inp = W.kgrouped_inputs()
    gk = inp["group_k"]
    qa, sa = oracle.cast_per_token(inp["a"], oracle.E4M3)
    qb, sb = oracle.cast_per_token(inp["b"], oracle.E4M3)
    out = dev(inp["out0"])
    te.te_fp8_kgrouped_wgrad(dev(qa), sdev(sa), E4, dev(qb), sdev(sb), E4, gk.tolist(), out, FULL)
    got = host(out).numpy()
    offs = np.concatenate([[0], np.cumsum(gk)])
    for g in range(sh["G"]):
        rows, cols = sample_idx(sh["M"], 8, 10 + g), sample_idx(sh["N"], 12, 20 + g)
        o, d = grid_entries(qa, sa, oracle.E4M3, qb, sb, oracle.E4M3, rows, cols, int(offs[g]), int(gk[g]))
        init = inp["out0"][g][np.ix_(rows, cols)]
        check_f32(got[g][np.ix_(rows, cols)], init.astype(np.float64) + o, np.abs(init) + d, f"expert {g}",
                  chain_gemm(gk[g], 1))
