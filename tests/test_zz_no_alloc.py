"""The entry point that allocates nothing (te_fp8_gemm_dgrad_deterministic_noalloc): its output is
the workspace form's, bit for bit, on two calls in a row (the second with a smaller input, so it
reads the static scratch the first call left behind), and it is held to the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import GELU_CHAIN, bf16_dev, chain_colsum, check_f32, dev, host, sdev

te = pytest.importorskip("fp8_linear_layer_amd")
pytestmark = pytest.mark.gpu

E4, E5 = te.TE_DTYPE_E4M3, te.TE_DTYPE_E5M2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    te.load_library()


def _case(M, N, K, seed):
    s = np.random.SeedSequence(seed).spawn(3)
    qa, sa = oracle.cast_per_token(W.normal_bf16(s[0], (M, K), 1e-3), oracle.E5M2)
    qb, sb = oracle.cast_per_token(W.normal_bf16(s[1], (N, K), 0.02), oracle.E4M3)
    z = W.normal_bf16(s[2], (M, N), 1.28)
    return qa, sa, qb, sb, z


@pytest.mark.parametrize("accum", [te.TE_ACCUM_FULL_FP32, te.TE_ACCUM_FAST])
def test_noalloc_matches_workspace_form_twice(accum):
    epi = te.TE_EPI_DGELU | te.TE_EPI_BGRAD
    for M, N, K, seed in ((1100, 1000, 512, 1), (300, 264, 256, 2)):     # second call smaller
        qa, sa, qb, sb, z = _case(M, N, K, seed)
        A, SA, B, SB, Z = dev(qa), sdev(sa), dev(qb), sdev(sb), bf16_dev(z)
        ld = N + 4 - N % 4
        bg_n = torch.full((N,), 7.0, dtype=torch.float32, device="cuda")
        dx_n = torch.full((M, ld), 5.0, dtype=torch.float32, device="cuda")[:, :N]
        te.te_fp8_gemm_dgrad_deterministic_noalloc(A, SA, E5, B, SB, E4, bg_n, dx_n, epilogue=epi, preact=Z,
                                                   dx_dtype=te.TE_DTYPE_F32, accum=accum)
        bg_w = torch.full((N,), 9.0, dtype=torch.float32, device="cuda")
        dx_w = torch.full((M, ld), 3.0, dtype=torch.float32, device="cuda")[:, :N]
        te.te_fp8_gemm_dgrad_deterministic(A, SA, E5, B, SB, E4, bg_w, epilogue=epi, preact=Z, dx=dx_w,
                                           dx_dtype=te.TE_DTYPE_F32, accum=accum)
        torch.cuda.synchronize()
        assert torch.equal(host(bg_n).view(torch.int32), host(bg_w).view(torch.int32)), (M, N, "bias grad")
        assert torch.equal(host(dx_n).view(torch.int32), host(dx_w).view(torch.int32)), (M, N, "dx")
        o, d = oracle.gemm_nt(qa, sa, oracle.E5M2, qb, sb, oracle.E4M3)
        _, _, db, dbm = oracle.dgrad_epilogue(o, d, z, bgrad=True)
        check_f32(host(bg_n).numpy(), db, dbm, "noalloc bias grad", chain_colsum(K, M, GELU_CHAIN))


def test_noalloc_rejects_outputs_beyond_its_scratch():
    lib = te.load_library()
    M, N = 8192, 16384 + 4       # one column group past the 8 MiB of column sums
    assert lib.te_fp8_dgrad_bgrad_workspace_bytes(M, N) > te.NOALLOC_SCRATCH_BYTES
    dy = torch.empty((M, 128), dtype=torch.uint8, device="cuda")
    wt = torch.empty((N, 128), dtype=torch.uint8, device="cuda")
    sd = torch.ones((1, te.scale_ld(M)), dtype=torch.float32, device="cuda")
    sw = torch.ones((1, te.scale_ld(N)), dtype=torch.float32, device="cuda")
    bg = torch.empty((N,), dtype=torch.float32, device="cuda")
    dx = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(te.TeFp8Error, match="static array"):
        te.te_fp8_gemm_dgrad_deterministic_noalloc(dy, sd, E5, wt, sw, E4, bg, dx, epilogue=te.TE_EPI_BGRAD)
