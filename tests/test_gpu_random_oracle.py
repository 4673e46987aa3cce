"""Seeded random ragged shapes against the fp64 oracle, on both GEMM kernels.

The fixed-shape parity tests pick their edges by hand.  These draw M in [1, 700), N in [8, 704)
(a multiple of 8, as the bias and the bf16 rows need), K a multiple of 128 up to 1024, from a fixed
seed, and check element by element against the oracle, with nothing written outside the outputs:
the forward with bias + GELU + saved pre-activation (FULL on IEEE scales, FAST on power-of-two
scales), the data gradient with dGELU and the ordered bias gradient, the weight gradient
(out += A B^T) and the quantising forward store (N rounded down to whole 1x128 groups).  The
grouped calls draw their group structure the same way: K-grouped weight gradients with 4-9 groups
of 0-5 blocks (empty groups must keep their output, -0.0 included), M-grouped forward and data
gradient with 3-8 blocks of 256 rows over 2-5 experts, some blocks skipped (their rows untouched)
and some experts without blocks (a zero bias gradient).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import (BIAS_CHAIN, GELU_CHAIN, GELU_LIP, bf16_dev, bf16_host_f64, chain_colsum, chain_gemm, check_bf16,
                    check_f32, check_quant, dev, host, scale_ld, sdev, shost)

te = pytest.importorskip("fp8_linear_layer_amd")
pytestmark = pytest.mark.gpu

E4, E5 = te.TE_DTYPE_E4M3, te.TE_DTYPE_E5M2
FULL, FAST = te.TE_ACCUM_FULL_FP32, te.TE_ACCUM_FAST


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    te.load_library()


@pytest.fixture(params=["wave", "persistent"])
def gemm_path(request, monkeypatch):
    monkeypatch.setenv("TE_FP8_GEMM_PATH", request.param)
    return request.param


def _shapes(n, seed):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 700)), int(rng.integers(1, 88)) * 8, int(rng.integers(1, 9)) * 128)
            for _ in range(n)]


SHAPES = _shapes(8, 355)


def cast(seed, rows, K, fmt, std, pow2):
    return oracle.cast_per_token(W.normal_bf16(np.random.SeedSequence(seed), (rows, K), std), fmt, pow2)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_random_fwd(M, N, K, gemm_path):
    epi = te.TE_EPI_BIAS | te.TE_EPI_GELU | te.TE_EPI_AUX_PREACT
    for accum, pow2 in ((FULL, False), (FAST, True)):
        qx, sx = cast(M * 3 + K, M, K, oracle.E4M3, 1.0, pow2)
        qw, sw = cast(N * 5 + K, N, K, oracle.E4M3, 0.05, pow2)
        b = W.normal_bf16(np.random.SeedSequence(N + 9), (N,), 0.1)
        o, d = oracle.gemm_nt(qx, sx, oracle.E4M3, qw, sw, oracle.E4M3)
        y, z, zmag = oracle.fwd_epilogue(o, d, b, True)
        ld = N + 8
        ybuf = torch.full((M + 1, ld), 77.0, dtype=torch.bfloat16, device="cuda")
        pbuf = torch.full((M + 1, ld), 55.0, dtype=torch.bfloat16, device="cuda")
        te.te_fp8_gemm_fwd(dev(qx), sdev(sx), E4, dev(qw), sdev(sw), E4, bias=bf16_dev(b), epilogue=epi,
                           y=ybuf[:M, :N], y_dtype=te.TE_DTYPE_BF16, preact=pbuf[:M, :N], accum=accum)
        torch.cuda.synchronize()
        yb, pb = host(ybuf), host(pbuf)
        what = f"fwd {M}x{N}x{K} {'fast-pow2' if pow2 else 'full'}"
        assert torch.all(yb[:M, N:] == 77.0) and torch.all(yb[M:] == 77.0), f"{what}: wrote outside y"
        assert torch.all(pb[:M, N:] == 55.0) and torch.all(pb[M:] == 55.0), f"{what}: wrote outside the preact"
        check_bf16(bf16_host_f64(yb[:M, :N]), y, zmag * GELU_LIP, f"{what}: y")
        check_bf16(bf16_host_f64(pb[:M, :N]), z, zmag, f"{what}: preact")


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_random_dgrad_dgelu_ordered_bias_grad(M, N, K, gemm_path):
    qa, sa = cast(M * 7 + K, M, K, oracle.E5M2, 1e-3, False)
    qb, sb = cast(N * 11 + K, N, K, oracle.E4M3, 0.02, False)
    zb = W.normal_bf16(np.random.SeedSequence(M + N), (M, N), 1.28)
    o, d = oracle.gemm_nt(qa, sa, oracle.E5M2, qb, sb, oracle.E4M3)
    D, Dm, db, dbm = oracle.dgrad_epilogue(o, d, zb, True)
    zpad = np.zeros((M, N + 8), np.uint16)
    zpad[:, :N] = zb
    dxbuf = torch.full((M + 1, N + 4), 9.0, dtype=torch.float32, device="cuda")
    bg = torch.full((N + 4,), 3.0, dtype=torch.float32, device="cuda")
    te.te_fp8_gemm_dgrad_deterministic(dev(qa), sdev(sa), E5, dev(qb), sdev(sb), E4, bg[:N],
                                       epilogue=te.TE_EPI_DGELU | te.TE_EPI_BGRAD, preact=bf16_dev(zpad)[:, :N],
                                       dx=dxbuf[:M, :N], dx_dtype=te.TE_DTYPE_F32, accum=FULL)
    torch.cuda.synchronize()
    xb, g = host(dxbuf).numpy(), host(bg).numpy()
    what = f"dgrad {M}x{N}x{K}"
    assert (xb[:M, N:] == 9.0).all() and (xb[M:] == 9.0).all(), f"{what}: wrote outside dx"
    assert (g[N:] == 3.0).all(), f"{what}: wrote past the bias gradient"
    check_f32(xb[:M, :N], D, Dm, f"{what}: dz", chain_gemm(K, GELU_CHAIN))
    check_f32(g[:N], db, dbm, f"{what}: ordered bias grad", chain_colsum(K, M, GELU_CHAIN))


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_random_wgrad(M, N, K, gemm_path):
    for accum, pow2 in ((FULL, False), (FAST, True)):
        qa, sa = cast(M * 13 + K, M, K, oracle.E5M2, 1e-3, pow2)
        qb, sb = cast(N * 17 + K, N, K, oracle.E4M3, 1.0, pow2)
        out0 = W.normal_f32(np.random.SeedSequence(M * N + K), (M, N))
        o, d = oracle.gemm_nt(qa, sa, oracle.E5M2, qb, sb, oracle.E4M3)
        want, mag = oracle.wgrad(o, d, out0)
        buf = torch.full((M + 1, N + 4), 1234.5, dtype=torch.float32, device="cuda")
        buf[:M, :N] = dev(out0)
        te.te_fp8_wgrad_accum(dev(qa), sdev(sa), E5, dev(qb), sdev(sb), E4, buf[:M, :N], accum)
        torch.cuda.synchronize()
        b = host(buf).numpy()
        what = f"wgrad {M}x{N}x{K} {'fast-pow2' if pow2 else 'full'}"
        assert (b[:M, N:] == 1234.5).all() and (b[M:] == 1234.5).all(), f"{what}: wrote outside out"
        check_f32(b[:M, :N], want, mag, what, chain_gemm(K, 1))


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_random_fwd_quant(M, N, K, gemm_path):
    N = max(128, N // 128 * 128)
    qx, sx = cast(M * 19 + K, M, K, oracle.E4M3, 1.0, False)
    qw, sw = cast(N * 23 + K, N, K, oracle.E4M3, 0.05, False)
    b = W.normal_bf16(np.random.SeedSequence(N + 29), (N,), 0.1)
    epi = te.TE_EPI_BIAS | te.TE_EPI_GELU
    o, d = oracle.gemm_nt(qx, sx, oracle.E4M3, qw, sw, oracle.E4M3)
    y, _, zmag = oracle.fwd_epilogue(o, d, b, True)
    X, SX, Wd, SW, Bd = dev(qx), sdev(sx), dev(qw), sdev(sw), bf16_dev(b)
    y32 = te.te_fp8_gemm_fwd(X, SX, E4, Wd, SW, E4, bias=Bd, epilogue=epi, y_dtype=te.TE_DTYPE_F32, accum=FULL)
    qbuf = torch.full((M, N + 16), 0xA5, dtype=torch.uint8, device="cuda")
    qs = torch.full((N // 128, scale_ld(M)), -3.0, dtype=torch.float32, device="cuda")
    te.te_fp8_gemm_fwd_quant(X, SX, E4, Wd, SW, E4, bias=Bd, epilogue=epi, q_dtype=E4, cast_flags=0,
                             q=qbuf[:, :N], q_scales=qs, accum=FULL)
    torch.cuda.synchronize()
    what = f"fwd quant {M}x{N}x{K}"
    qh, sh = host(qbuf).numpy(), host(qs).numpy()
    assert (qh[:, N:] == 0xA5).all(), f"{what}: wrote past N"
    assert (sh[:, M:] == -3.0).all(), f"{what}: wrote into the scale padding"
    # the codes are the cast of the kernel's own fp32 result, bit for bit, and held to the fp64 oracle
    qo, so = oracle.cast_per_token_f32(host(y32).numpy(), oracle.E4M3, False)
    assert np.array_equal(qh[:, :N], qo), f"{what}: codes differ from the cast of the fp32 forward"
    s = shost(qs, M)
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32)), f"{what}: scales differ"
    check_quant(qh[:, :N], s, oracle.E4M3, y, zmag * GELU_LIP, what, chain_gemm(K, BIAS_CHAIN + GELU_CHAIN))


def _kgroups(seed):
    """4-9 groups of 0-5 blocks of 128 (at least one non-empty), M and N ragged."""
    rng = np.random.default_rng(seed)
    gk = rng.integers(1, 6, int(rng.integers(4, 10))) * 128
    gk[rng.random(gk.size) < 0.25] = 0
    gk[int(rng.integers(0, gk.size))] = 256
    return gk.astype(np.int64), int(rng.integers(1, 400)), int(rng.integers(1, 50)) * 8


@pytest.mark.parametrize("seed", [61, 62, 63, 64])
def test_random_kgrouped(seed, gemm_path):
    gk, M, N = _kgroups(seed)
    S = int(gk.sum())
    for accum, pow2 in ((FULL, False), (FAST, True)):
        qa, sa = cast(seed * 3, M, S, oracle.E5M2, 1e-3, pow2)
        qb, sb = cast(seed * 3 + 1, N, S, oracle.E4M3, 1.0, pow2)
        init = W.normal_f32(np.random.SeedSequence(seed * 3 + 2), (gk.size, M, N))
        init[:, 0, 0] = -0.0
        want, mag = oracle.kgrouped_wgrad(qa, sa, oracle.E5M2, qb, sb, oracle.E4M3, gk, init)
        out = dev(init)
        te.te_fp8_kgrouped_wgrad(dev(qa), sdev(sa), E5, dev(qb), sdev(sb), E4, gk.tolist(), out, accum)
        got = host(out).numpy()
        what = f"kgrouped {gk.tolist()} {M}x{N} {'fast-pow2' if pow2 else 'full'}"
        for g in range(gk.size):
            if gk[g] == 0:
                assert np.array_equal(got[g].view(np.uint32), init[g].view(np.uint32)), f"{what}: empty group {g}"
            else:
                check_f32(got[g], want[g], mag[g], f"{what}: group {g}", chain_gemm(int(gk[g]), 1))


def _mblocks(seed):
    """3-8 blocks of 256 rows over G = 2-5 experts, about one in six skipped (-1); N ragged."""
    rng = np.random.default_rng(seed)
    G = int(rng.integers(2, 6))
    blocks = rng.integers(0, G, int(rng.integers(3, 9))).astype(np.int32)
    blocks[rng.random(blocks.size) < 1 / 6] = -1
    blocks[int(rng.integers(0, blocks.size))] = int(rng.integers(0, G))
    return G, blocks, int(rng.integers(1, 60)) * 8, int(rng.integers(1, 7)) * 128


@pytest.mark.parametrize("seed", [71, 72, 73, 74])
def test_random_mgrouped_fwd_and_dgrad(seed, gemm_path):
    G, blocks, N, K = _mblocks(seed)
    M = 256 * blocks.size
    live = np.repeat(blocks >= 0, 256)
    what = f"mgrouped G={G} {blocks.tolist()} N={N} K={K}"
    qx, sx = cast(seed * 5, M, K, oracle.E4M3, 1.0, False)
    wts = [cast(seed * 5 + 1 + e, N, K, oracle.E4M3, 0.05, False) for e in range(G)]
    qw, sw = np.stack([w[0] for w in wts]), np.stack([w[1] for w in wts])
    wq, wsd = dev(qw), torch.stack([sdev(sw[e]) for e in range(G)]).contiguous()
    bmap = torch.from_numpy(blocks).cuda()
    # forward: bias + GELU, bf16 y and pre-activation
    b = W.normal_bf16(np.random.SeedSequence(seed * 5 + 9), (G, N), 0.1)
    y, z, zmag = oracle.mgrouped_fwd(qx, sx, oracle.E4M3, qw, sw, oracle.E4M3, blocks, b, True)
    ybuf = torch.full((M, N + 8), 77.0, dtype=torch.bfloat16, device="cuda")
    pbuf = torch.full((M, N + 8), 55.0, dtype=torch.bfloat16, device="cuda")
    te.te_fp8_mgrouped_gemm_fwd(dev(qx), sdev(sx), E4, wq, wsd, E4, bmap, bias=bf16_dev(b),
                                epilogue=te.TE_EPI_BIAS | te.TE_EPI_GELU | te.TE_EPI_AUX_PREACT, y=ybuf[:, :N],
                                y_dtype=te.TE_DTYPE_BF16, preact=pbuf[:, :N], accum=FULL)
    torch.cuda.synchronize()
    yb, pb = host(ybuf), host(pbuf)
    dead = torch.from_numpy(~live)
    assert torch.all(yb[:, N:] == 77.0) and torch.all(yb[dead] == 77.0), f"{what}: y written outside live rows"
    assert torch.all(pb[:, N:] == 55.0) and torch.all(pb[dead] == 55.0), f"{what}: preact written outside"
    check_bf16(bf16_host_f64(yb[:, :N])[live], y[live], zmag[live] * GELU_LIP, f"{what}: y")
    check_bf16(bf16_host_f64(pb[:, :N])[live], z[live], zmag[live], f"{what}: preact")
    # data gradient: dGELU on the pre-activation, per-expert ordered bias gradient, fp32 dx
    qa, sa = cast(seed * 5 + 7, M, K, oracle.E5M2, 1e-3, False)
    zb = W.normal_bf16(np.random.SeedSequence(seed * 5 + 8), (M, N), 1.28)
    D, Dm, db, dbm = oracle.mgrouped_dgrad(qa, sa, oracle.E5M2, qw, sw, oracle.E4M3, blocks, zb)
    zpad = np.zeros((M, N + 8), np.uint16)
    zpad[:, :N] = zb
    dxbuf = torch.full((M, N + 4), 9.0, dtype=torch.float32, device="cuda")
    bg = torch.full((G * N,), 3.0, dtype=torch.float32, device="cuda")
    te.te_fp8_mgrouped_gemm_dgrad_deterministic(dev(qa), sdev(sa), E5, wq, wsd, E4, bmap, bg,
                                                epilogue=te.TE_EPI_DGELU | te.TE_EPI_BGRAD,
                                                preact=bf16_dev(zpad)[:, :N], dx=dxbuf[:, :N],
                                                dx_dtype=te.TE_DTYPE_F32, accum=FULL)
    torch.cuda.synchronize()
    xb, g = host(dxbuf).numpy(), host(bg).numpy().reshape(G, N)
    assert (xb[:, N:] == 9.0).all() and (xb[~live] == 9.0).all(), f"{what}: dx written outside live rows"
    check_f32(xb[:, :N][live], D[live], Dm[live], f"{what}: dz", chain_gemm(K, GELU_CHAIN))
    used = np.isin(np.arange(G), blocks)
    assert (g[~used] == 0).all(), f"{what}: an expert without blocks must get a zero bias gradient"
    if used.any():
        check_f32(g[used], db[used], dbm[used], f"{what}: per-expert bias grad", chain_colsum(K, M, GELU_CHAIN))
