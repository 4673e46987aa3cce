"""The library under HIP graph capture: a training step's calls (cast, fprop with bias + GELU + saved
pre-activation, dgrad with dGELU + bias gradient, wgrad out +=, the K-grouped wgrad with device-side
sizes) recorded once and replayed several times, each replay checked bit for bit against the same
calls run eagerly.  The library allocates nothing, never synchronises and clears the bias gradient
with a kernel (no memset node), so every call can be captured."""
import numpy as np
import pytest
import torch

import workloads as W
from parity import bf16_dev

te = pytest.importorskip("fp8_linear_layer_amd")
pytestmark = pytest.mark.gpu

E4, E5 = te.TE_DTYPE_E4M3, te.TE_DTYPE_E5M2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    te.load_library()


def test_training_step_replays_match_eager():
    T, IN, OUT = 512, 384, 640                       # tokens, in features, out features
    s = W.spawn(31, 6)
    x = bf16_dev(W.normal_bf16(s[0], (T, IN)))
    w = bf16_dev(W.normal_bf16(s[1], (OUT, IN), 0.05))
    b = bf16_dev(W.normal_bf16(s[2], (OUT,), 0.1))
    dy = bf16_dev(W.normal_bf16(s[3], (T, OUT), 1e-2))
    w1t = bf16_dev(W.normal_bf16(s[4], (IN, OUT), 0.05))  # a downstream layer's W^T for the dgrad
    wg = torch.from_numpy(W.normal_f32(s[5], (OUT, IN))).cuda()
    gk = torch.tensor([128, 0, 256, 128], dtype=torch.int64, device="cuda")   # sums to T

    def step(o):
        qx, sx, qxt, sxt = te.te_cast_fp8_per_token_transpose(x, E4, q=o["qx"], scales=o["sx"], qt=o["qxt"],
                                                              scales_t=o["sxt"])
        qw, sw = te.te_cast_fp8_per_token(w, E4, q=o["qw"], scales=o["sw"])
        te.te_fp8_gemm_fwd(qx, sx, E4, qw, sw, E4, bias=b, epilogue=te.TE_EPI_BIAS | te.TE_EPI_GELU |
                           te.TE_EPI_AUX_PREACT, y=o["y"], preact=o["z"], accum=te.TE_ACCUM_FAST)
        _, _, qdyt, sdyt = te.te_cast_fp8_per_token_transpose(dy, E5, rowwise=False, qt=o["qdyt"], scales_t=o["sdyt"])
        qdy, sdy = te.te_cast_fp8_per_token(dy, E5, q=o["qdy"], scales=o["sdy"])
        qwt, swt = te.te_cast_fp8_per_token(w1t, E4, q=o["qwt"], scales=o["swt"])
        te.te_fp8_gemm_dgrad(qdy, sdy, E5, qwt, swt, E4, epilogue=te.TE_EPI_DGELU | te.TE_EPI_BGRAD,
                             preact=o["z2"], bias_grad=o["db"], dx=o["dx"], accum=te.TE_ACCUM_FULL_FP32)
        te.te_fp8_wgrad_accum(qdyt, sdyt, E5, qxt, sxt, E4, o["wgrad"], te.TE_ACCUM_FULL_FP32)
        te.te_fp8_kgrouped_wgrad_device_sizes(qdyt, sdyt, E5, qxt, sxt, E4, gk, o["kg"], te.TE_ACCUM_FULL_FP32)

    def buffers():
        o = {
            "qx": torch.empty((T, IN), dtype=torch.uint8, device="cuda"),
            "sx": torch.empty((IN // 128, te.scale_ld(T)), dtype=torch.float32, device="cuda"),
            "qxt": torch.empty((IN, T), dtype=torch.uint8, device="cuda"),
            "sxt": torch.empty((T // 128, te.scale_ld(IN)), dtype=torch.float32, device="cuda"),
            "qw": torch.empty((OUT, IN), dtype=torch.uint8, device="cuda"),
            "sw": torch.empty((IN // 128, te.scale_ld(OUT)), dtype=torch.float32, device="cuda"),
            "y": torch.empty((T, OUT), dtype=torch.bfloat16, device="cuda"),
            "z": torch.empty((T, OUT), dtype=torch.bfloat16, device="cuda"),
            "qdyt": torch.empty((OUT, T), dtype=torch.uint8, device="cuda"),
            "sdyt": torch.empty((T // 128, te.scale_ld(OUT)), dtype=torch.float32, device="cuda"),
            "qdy": torch.empty((T, OUT), dtype=torch.uint8, device="cuda"),
            "sdy": torch.empty((OUT // 128, te.scale_ld(T)), dtype=torch.float32, device="cuda"),
            "qwt": torch.empty((IN, OUT), dtype=torch.uint8, device="cuda"),
            "swt": torch.empty((OUT // 128, te.scale_ld(IN)), dtype=torch.float32, device="cuda"),
            "z2": torch.from_numpy(W.bf16_bits_to_f32(W.normal_bf16(np.random.SeedSequence(77), (T, IN), 1.28)))
                       .to(torch.bfloat16).cuda(),
            "db": torch.empty((IN,), dtype=torch.float32, device="cuda"),
            "dx": torch.empty((T, IN), dtype=torch.bfloat16, device="cuda"),
            "wgrad": wg.clone(),
            "kg": torch.zeros((4, OUT, IN), dtype=torch.float32, device="cuda"),
        }
        return o

    # eager reference: three steps (wgrad and the K-grouped outputs accumulate)
    ref = buffers()
    eager = []
    for _ in range(3):
        step(ref)
        torch.cuda.synchronize()
        eager.append({k: v.clone() for k, v in ref.items()})

    g_out = buffers()
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(g_out)
    torch.cuda.synchronize()
    # capture does not run the kernels: restore the accumulators before the first replay
    g_out["wgrad"].copy_(wg)
    g_out["kg"].zero_()
    torch.cuda.synchronize()
    for r in range(3):
        graph.replay()
        torch.cuda.synchronize()
        _ = torch.ones(1000, device="cuda").sum().item()   # eager work between replays
        for k, v in g_out.items():
            if k == "db":
                # atomic order may differ between runs: compare within fp32 summation error
                assert torch.allclose(v, eager[r][k], rtol=1e-5, atol=1e-6), f"replay {r}: {k}"
            else:
                assert torch.equal(v.view(torch.uint8) if v.dtype != torch.uint8 else v,
                                   eager[r][k].view(torch.uint8) if v.dtype != torch.uint8 else eager[r][k]), \
                    f"replay {r}: {k}"


def test_quantising_and_deterministic_calls_replay_match_eager():
    """The two-layout quantising forward, the deterministic dense and M-grouped data gradients
    (workspace-based bias gradients) under capture: every replay bit-identical to the eager calls."""
    T, IN, OUT, G = 512, 384, 640, 2
    s = W.spawn(41, 6)
    qx, sx = te.te_cast_fp8_per_token(bf16_dev(W.normal_bf16(s[0], (T, IN))), E4)
    qw, sw = te.te_cast_fp8_per_token(bf16_dev(W.normal_bf16(s[1], (OUT, IN), 0.05)), E4)
    b = bf16_dev(W.normal_bf16(s[2], (OUT,), 0.1))
    qdy, sdy = te.te_cast_fp8_per_token(bf16_dev(W.normal_bf16(s[3], (T, OUT), 1e-2)), E5)
    qwt, swt = te.te_cast_fp8_per_token(bf16_dev(W.normal_bf16(s[4], (G * IN, OUT), 0.05)), E4)
    z = bf16_dev(W.normal_bf16(s[5], (T, IN), 1.28))
    qwt_g = qwt.view(G, IN, OUT)
    swt_g = swt.view(OUT // 128, G, IN).permute(1, 0, 2).contiguous()
    blocks = torch.tensor([1, 0], dtype=torch.int32, device="cuda")
    lib = te.load_library()
    DB = te.TE_EPI_DGELU | te.TE_EPI_BGRAD

    def buffers():
        return {
            "q": torch.empty((T, OUT), dtype=torch.uint8, device="cuda"),
            "qs": torch.empty((OUT // 128, te.scale_ld(T)), dtype=torch.float32, device="cuda"),
            "qt": torch.empty((OUT, T), dtype=torch.uint8, device="cuda"),
            "qts": torch.empty((T // 128, te.scale_ld(OUT)), dtype=torch.float32, device="cuda"),
            "dx": torch.empty((T, IN), dtype=torch.bfloat16, device="cuda"),
            "db": torch.empty((IN,), dtype=torch.float32, device="cuda"),
            "ws": torch.empty((lib.te_fp8_dgrad_bgrad_workspace_bytes(T, IN),), dtype=torch.uint8, device="cuda"),
            "dxg": torch.empty((T, IN), dtype=torch.bfloat16, device="cuda"),
            "dbg": torch.empty((G * IN,), dtype=torch.float32, device="cuda"),
            "wsg": torch.empty((lib.te_fp8_dgrad_bgrad_workspace_bytes(T, IN),), dtype=torch.uint8, device="cuda"),
        }

    def step(o):
        te.te_fp8_gemm_fwd_quant(qx, sx, E4, qw, sw, E4, bias=b, epilogue=te.TE_EPI_BIAS | te.TE_EPI_GELU,
                                 q=o["q"], q_scales=o["qs"], transposed=True, qt=o["qt"], qt_scales=o["qts"],
                                 accum=te.TE_ACCUM_FAST)
        te.te_fp8_gemm_dgrad_deterministic(qdy, sdy, E5, qwt[:IN], swt[:, :te.scale_ld(IN)].contiguous(), E4,
                                           o["db"], epilogue=DB, preact=z, workspace=o["ws"], dx=o["dx"])
        te.te_fp8_mgrouped_gemm_dgrad_deterministic(qdy, sdy, E5, qwt_g, swt_g, E4, blocks, o["dbg"], epilogue=DB,
                                                    preact=z, workspace=o["wsg"], dx=o["dxg"])

    ref = buffers()
    step(ref)
    torch.cuda.synchronize()
    g_out = buffers()
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(g_out)
    torch.cuda.synchronize()
    for r in range(3):
        for k in ("ws", "wsg"):
            g_out[k].fill_(0xFF)                       # the workspaces start as garbage every time
        graph.replay()
        torch.cuda.synchronize()
        _ = torch.ones(1000, device="cuda").sum().item()
        for k in ("q", "qs", "qt", "qts", "dx", "db", "dxg", "dbg"):
            v, e = g_out[k], ref[k]
            if k in ("qs", "qts"):
                rows = T if k == "qs" else OUT
                v, e = v[:, :rows], e[:, :rows]
            assert torch.equal(v.contiguous().view(torch.uint8), e.contiguous().view(torch.uint8)), f"replay {r}: {k}"
