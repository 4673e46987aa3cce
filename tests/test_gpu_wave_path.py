"""The wave-tile GEMM path (products with few 256 x 256 tiles) against the persistent one.

Both kernels take the same fragments, promote in the same order (FULL) or chain through the matrix
core (FAST on power-of-two scales) and share the epilogue, so on the same inputs every output that is
not summed with atomics must come out bit for bit the same; the oracle parity of each path is
covered by test_gpu_gemm.py, which runs its small products on both.  Shapes: the tiny Linear
(256 x 256 x 512, one tile), one wave tile exactly, one element past it in both dimensions, and a
ragged product spanning two tiles each way; then the grouped calls (K-grouped with host and device
sizes, M-grouped forward and deterministic data gradient).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import bf16_dev, dev, host, sdev

te = pytest.importorskip("fp8_linear_layer_amd")
pytestmark = pytest.mark.gpu

E4, E5 = te.TE_DTYPE_E4M3, te.TE_DTYPE_E5M2
FULL, FAST = te.TE_ACCUM_FULL_FP32, te.TE_ACCUM_FAST
SHAPES = [(256, 256, 512), (64, 128, 256), (65, 129, 128), (300, 264, 384)]
POL = [(FULL, False), (FAST, True), (FAST, False)]
PID = ["full", "fast-pow2", "fast-ieee"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    te.load_library()


def operand(seed, rows, K, fmt, std, pow2):
    bits = W.normal_bf16(np.random.SeedSequence(seed), (rows, K), std)
    q, s = oracle.cast_per_token(bits, fmt, pow2)
    return dev(q), sdev(s)


def both(monkeypatch, run):
    """run() on the wave path, then on the persistent one; each returns a list of tensors."""
    out = {}
    for path in ("wave", "persistent"):
        monkeypatch.setenv("TE_FP8_GEMM_PATH", path)
        out[path] = [host(t).contiguous() for t in run()]
        torch.cuda.synchronize()
    return out["wave"], out["persistent"]


def padded(M, N, dtype, fill=0.0):
    """An [M, N] view of a buffer whose rows are padded to 16 bytes (the ABI's stride rule)."""
    per = 16 // torch.tensor([], dtype=dtype).element_size()
    return torch.full((M, (N + per - 1) // per * per), fill, dtype=dtype, device="cuda")[:, :N]


def same_bits(a, b, what):
    for i, (x, y) in enumerate(zip(a, b)):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"{what}: output {i} differs between the paths"


@pytest.mark.parametrize("accum,pow2", POL, ids=PID)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_wgrad_paths_agree(monkeypatch, accum, pow2, M, N, K):
    A, SA = operand(M + 1, M, K, oracle.E4M3, 1.0, pow2)
    B, SB = operand(N + 2, N, K, oracle.E4M3, 1.0, pow2)
    out0 = dev(W.normal_f32(np.random.SeedSequence(M + N + 3), (M, N)))

    def run():
        out = padded(M, N, torch.float32)
        out.copy_(out0)
        te.te_fp8_wgrad_accum(A, SA, E4, B, SB, E4, out, accum)
        return [out]
    same_bits(*both(monkeypatch, run), "wgrad")


@pytest.mark.parametrize("accum,pow2", POL, ids=PID)
@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("ydt", [te.TE_DTYPE_BF16, te.TE_DTYPE_F32])
def test_fwd_paths_agree(monkeypatch, accum, pow2, M, N, K, ydt):
    X, SX = operand(M + 11, M, K, oracle.E4M3, 1.0, pow2)
    Wt, SW = operand(N + 12, N, K, oracle.E4M3, 0.02, pow2)
    b = bf16_dev(W.normal_bf16(np.random.SeedSequence(N + 13), (N,), 0.1))
    epi = te.TE_EPI_BIAS | te.TE_EPI_GELU | te.TE_EPI_AUX_PREACT

    def run():
        z = padded(M, N, torch.bfloat16)
        y = padded(M, N, torch.bfloat16 if ydt == te.TE_DTYPE_BF16 else torch.float32)
        te.te_fp8_gemm_fwd(X, SX, E4, Wt, SW, E4, bias=b, epilogue=epi, y=y, y_dtype=ydt, preact=z, accum=accum)
        return [y, z]
    same_bits(*both(monkeypatch, run), "fwd")


@pytest.mark.parametrize("accum,pow2", POL, ids=PID)
@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (300, 384, 256)])
def test_fwd_quant_paths_agree(monkeypatch, accum, pow2, M, N, K):
    X, SX = operand(M + 21, M, K, oracle.E4M3, 1.0, pow2)
    Wt, SW = operand(N + 22, N, K, oracle.E4M3, 0.02, pow2)
    b = bf16_dev(W.normal_bf16(np.random.SeedSequence(N + 23), (N,), 0.1))

    def run():
        q, s = te.te_fp8_gemm_fwd_quant(X, SX, E4, Wt, SW, E4, bias=b, epilogue=te.TE_EPI_BIAS | te.TE_EPI_GELU,
                                        accum=accum)
        return [q, s[:, :M]]
    same_bits(*both(monkeypatch, run), "fwd quant")


@pytest.mark.parametrize("accum,pow2", POL, ids=PID)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_dgrad_paths_agree(monkeypatch, accum, pow2, M, N, K):
    """dX (fp32, after dGELU) and the deterministic bias gradient, whose workspace rows the wave
    path fills per wave place (zero for a place past M) exactly as the persistent kernel's waves."""
    D, SD = operand(M + 31, M, K, oracle.E5M2, 1e-3, pow2)
    Wt, SW = operand(N + 32, N, K, oracle.E4M3, 0.02, pow2)
    z = padded(M, N, torch.bfloat16)
    z.copy_(bf16_dev(W.normal_bf16(np.random.SeedSequence(M + 33), (M, N), 1.28)))
    epi = te.TE_EPI_DGELU | te.TE_EPI_BGRAD

    def run():
        bg = torch.full((N,), 7.0, dtype=torch.float32, device="cuda")
        dx = padded(M, N, torch.float32)
        te.te_fp8_gemm_dgrad_deterministic(D, SD, E5, Wt, SW, E4, bg, epilogue=epi, preact=z, dx=dx,
                                           dx_dtype=te.TE_DTYPE_F32, accum=accum)
        return [dx, bg]
    same_bits(*both(monkeypatch, run), "dgrad")


def _random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.integers(1, 700))
        N = int(rng.integers(1, 700))
        K = 128 * int(rng.integers(1, 9))
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", _random_shapes(16, 2026))
def test_random_shapes_paths_agree(monkeypatch, M, N, K):
    """Seeded random ragged shapes (M, N in [1, 700), K a multiple of 128 up to 1024): the
    wave-tile and persistent kernels agree bit for bit on the weight gradient under FULL and FAST
    (power-of-two scales), and on the forward with bias + GELU."""
    for accum, pow2 in ((FULL, False), (FAST, True)):
        A, SA = operand(M * 7 + K, M, K, oracle.E4M3, 1.0, pow2)
        B, SB = operand(N * 11 + K, N, K, oracle.E4M3, 1.0, pow2)
        out0 = dev(W.normal_f32(np.random.SeedSequence(M + 3 * N), (M, N)))

        def run_w():
            out = padded(M, N, torch.float32)
            out.copy_(out0)
            te.te_fp8_wgrad_accum(A, SA, E4, B, SB, E4, out, accum)
            return [out]
        same_bits(*both(monkeypatch, run_w), f"wgrad {M}x{N}x{K}")
    X, SX = operand(M + 5, M, K, oracle.E4M3, 1.0, False)
    Wt, SW = operand(N + 6, N, K, oracle.E4M3, 0.02, False)
    b = bf16_dev(W.normal_bf16(np.random.SeedSequence(N + 7), (N,), 0.1))

    def run_f():
        y = padded(M, N, torch.bfloat16)
        te.te_fp8_gemm_fwd(X, SX, E4, Wt, SW, E4, bias=b, epilogue=te.TE_EPI_BIAS | te.TE_EPI_GELU, y=y,
                           accum=FULL)
        return [y]
    same_bits(*both(monkeypatch, run_f), f"fwd {M}x{N}x{K}")


@pytest.mark.parametrize("accum,pow2", POL, ids=PID)
@pytest.mark.parametrize("sizes", ["host", "device"])
def test_kgrouped_paths_agree(monkeypatch, accum, pow2, sizes):
    """K-grouped weight gradient (empty groups among them, one output holding -0.0 that an empty
    group must leave as it is): each tile's group, contraction range and output come from the same
    tile context on both kernels."""
    gk = np.array([256, 0, 384, 128, 0, 512], np.int64)
    M, N, S = 300, 200, int(gk.sum())
    A, SA = operand(71, M, S, oracle.E4M3, 1.0, pow2)
    B, SB = operand(72, N, S, oracle.E4M3, 1.0, pow2)
    init = W.normal_f32(np.random.SeedSequence(73), (len(gk), M, N))
    init[1, :5, :3] = -0.0
    gkd = torch.from_numpy(gk).cuda()

    def run():
        out = dev(init)
        if sizes == "host":
            te.te_fp8_kgrouped_wgrad(A, SA, E4, B, SB, E4, gk.tolist(), out, accum)
        else:
            te.te_fp8_kgrouped_wgrad_device_sizes(A, SA, E4, B, SB, E4, gkd, out, accum)
        return [out]
    wave, pers = both(monkeypatch, run)
    same_bits(wave, pers, "kgrouped")
    assert np.array_equal(wave[0][1].numpy().view(np.uint32), init[1].view(np.uint32)), "empty group touched"


def _mgrouped_operands(seed, G, blocks, N, K, fx, std, pow2):
    M = 256 * len(blocks)
    X, SX = operand(seed, M, K, fx, std, pow2)
    ws = [W.normal_bf16(np.random.SeedSequence(seed + 1 + e), (N, K), 0.02) for e in range(G)]
    cw = [oracle.cast_per_token(w, oracle.E4M3, pow2) for w in ws]
    Wq = dev(np.stack([c[0] for c in cw]))
    Ws = torch.stack([sdev(c[1]) for c in cw]).contiguous()
    return M, X, SX, Wq, Ws


@pytest.mark.parametrize("accum,pow2", POL, ids=PID)
def test_mgrouped_fwd_paths_agree(monkeypatch, accum, pow2):
    """M-grouped forward with bias + GELU + pre-activation store; blocks on three experts, one
    skipped (-1) and one out of range (5): its rows stay untouched on both kernels."""
    blocks = np.array([2, 0, -1, 2, 1, 5], np.int32)
    G, N, K = 3, 296, 384      # (a bias row per expert must stay 16-byte aligned: N a multiple of 8)
    M, X, SX, Wq, Ws = _mgrouped_operands(81, G, blocks, N, K, oracle.E4M3, 1.0, pow2)
    b = bf16_dev(W.normal_bf16(np.random.SeedSequence(89), (G, N), 0.1))
    mb = torch.from_numpy(blocks).cuda()
    epi = te.TE_EPI_BIAS | te.TE_EPI_GELU | te.TE_EPI_AUX_PREACT

    def run():
        y = padded(M, N, torch.bfloat16, 7.0)
        z = padded(M, N, torch.bfloat16, 5.0)
        te.te_fp8_mgrouped_gemm_fwd(X, SX, E4, Wq, Ws, E4, mb, bias=b, epilogue=epi, y=y, preact=z, accum=accum)
        return [y, z]
    wave, pers = both(monkeypatch, run)
    same_bits(wave, pers, "mgrouped fwd")
    dead = torch.from_numpy(np.repeat((blocks < 0) | (blocks >= G), 256))
    assert torch.all(wave[0][dead] == 7.0) and torch.all(wave[1][dead] == 5.0), "a skipped block was written"


@pytest.mark.parametrize("accum,pow2", POL, ids=PID)
def test_mgrouped_dgrad_deterministic_paths_agree(monkeypatch, accum, pow2):
    """M-grouped data gradient through GELU' with the deterministic per-expert bias gradients: dX
    and every expert's bias gradient (expert 1 has no block: zeros) agree bit for bit."""
    blocks = np.array([2, 0, -1, 2, 0], np.int32)
    G, N, K = 3, 264, 256
    M, D, SD, Wq, Ws = _mgrouped_operands(91, G, blocks, N, K, oracle.E5M2, 1e-3, pow2)
    z = padded(M, N, torch.bfloat16)
    z.copy_(bf16_dev(W.normal_bf16(np.random.SeedSequence(99), (M, N), 1.28)))
    mb = torch.from_numpy(blocks).cuda()
    epi = te.TE_EPI_DGELU | te.TE_EPI_BGRAD

    def run():
        bg = torch.full((G * N,), 3.0, dtype=torch.float32, device="cuda")
        dx = padded(M, N, torch.float32, 9.0)
        te.te_fp8_mgrouped_gemm_dgrad_deterministic(D, SD, E5, Wq, Ws, E4, mb, bg, epilogue=epi, preact=z, dx=dx,
                                                    dx_dtype=te.TE_DTYPE_F32, accum=accum)
        return [dx, bg]
    wave, pers = both(monkeypatch, run)
    same_bits(wave, pers, "mgrouped dgrad")
    assert torch.all(wave[1].reshape(G, N)[1] == 0), "an expert without blocks must get a zero bias gradient"
