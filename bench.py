"""Benchmark of the scaled-FP8 Linear-layer hot path on one MI355X.

One step = the dense weight-gradient path at 7168 x 2112 x 4096: per-token
1x128 e4m3 cast of both bf16 operands (dY^T [7168, 4096] and X^T [2112, 4096],
one batched launch) followed by the block-scaled FP8 GEMM that accumulates out[7168, 2112] += A B^T
in fp32 with full-precision promotion.  Inputs are seeded synthetic bf16
N(0, 1) already resident in HBM; the fp32 accumulator is pre-filled N(0, 1).

Printed: one JSON line with the whole-step throughput (2 M N K flop per step),
the GEMM kernel's roofline fraction against the FP8 dense matrix-core peak
(kernel time from HIP events on the launch stream), the oracle's CPU
throughput on a bounded sample, and per-kernel timings of the other
workloads (the tiny 256 x 256 x 512 fprop and wgrad calls, fprop with
bias+GELU at 8192 x 14336 x 4096 in both accumulation
policies and with the quantising store, the fused cast + cast-transpose of the activation, dgrad at
8192 x 4096 x 14336 and its dGELU+bias-grad form (also with the
deterministic bias gradient, and storing e5m2 dZ),
the e5m2 cast of the gradient, the dense weight gradient fed from token-major sources through
the cast-transpose, the 8-expert K-grouped wgrad with its group sizes on
the host and on the device, and the 8-expert M-grouped forward).
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_FP8_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 matrix-core peak
HBM_PEAK_GBS = 8000.0
PAGES_TFLOPS_SAME_SHAPE = 920.0  # dense wgrad 7168x2112x4096 as published (hardware not named)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # (the clocks settle after ~300 steps, ~35 ms of this step; 500 timed steps take ~55 ms)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=20, help="back-to-back GEMM launches timed for kernel_ms")
    ap.add_argument("--cpu-rows", type=int, default=7168, help="rows of the oracle's CPU sample")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="minimum CPU time of the oracle sample")
    ap.add_argument("--cold-steps", type=int, default=30, help="steps timed after a cache flush each")
    ap.add_argument("--case", default=None, help="run one named workload alone (see GROUPS) and print its time")
    ap.add_argument("--reps", type=int, default=20, help="launches of --case")
    ap.add_argument("--breakdown-rounds", type=int, default=20)
    ap.add_argument("--ref-copy", action="store_true",
                    help="first run three plain 1 GiB device copies (reference for HBM byte counters)")
    return ap.parse_args()


def kernel_hash():
    """Hash of the kernel sources with comments and blank space removed, so that an edit of a
    comment does not orphan counters taken on the same code."""
    import re
    h = hashlib.sha256()
    for f in ("gemm.hip", "cast.hip"):
        with open(os.path.join(ROOT, "fp8_linear_layer_amd", "csrc", f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel_key: str):
    """HBM bytes per launch of the GEMM kernel from the committed PMC summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_hash():
        return None
    entry = rec.get("kernels", {}).get(kernel_key)
    return None if entry is None else entry.get("hbm_bytes_per_launch")


def timed(fn, reps, warm=3, rounds=3):
    """Kernel time of fn (one launch): `reps` back-to-back launches between one
    event pair on the launch stream, divided by reps (an event pair around a
    single launch would also count the dispatch gap in front of it).  Median
    and minimum over `rounds` such runs."""
    import torch
    for _ in range(warm):
        fn()
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(rounds):
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st.record(stream)
        for _ in range(reps):
            fn()
        en.record(stream)
        en.synchronize()
        times.append(st.elapsed_time(en) / reps)
    return float(np.median(times)), float(np.min(times))


def timed_interleaved(fns, reps, rounds, warm=3):
    """The kernel times of several launches measured in turn: each round times `reps` back-to-back
    launches of every fn (one event pair each), in the same order, so a drifting clock affects them
    alike.  Returns name -> list of per-launch times (ms), one per round."""
    import torch
    for fn in fns.values():
        for _ in range(warm):
            fn()
    stream = torch.cuda.current_stream()
    out = {k: [] for k in fns}
    for _ in range(rounds):
        evs = []
        for k, fn in fns.items():
            st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            st.record(stream)
            for _ in range(reps):
                fn()
            en.record(stream)
            evs.append((k, st, en))
        evs[-1][2].synchronize()
        for k, st, en in evs:
            out[k].append(st.elapsed_time(en) / reps)
    return out


class Case:
    """One timed launch: fn, its flop (GEMMs) or algorithmic bytes (HBM-bound kernels)."""

    def __init__(self, fn, flop=None, nbytes=None, note=None):
        self.fn, self.flop, self.nbytes, self.note = fn, flop, nbytes, note


def _randn(torch, g, shape, std, seed):
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device="cuda", dtype=torch.float32) * std).to(torch.bfloat16)


def group_tiny(te, torch, g):
    """256 x 256 x 512: bias + GELU fprop (fp32 out) and the wgrad += call on the same operands."""
    E4 = te.TE_DTYPE_E4M3
    xt, wt_, bt = _randn(torch, g, (256, 512), 1.0, 21), _randn(torch, g, (256, 512), 1.0, 22), \
        _randn(torch, g, (256,), 0.1, 23)
    qxt, sxt = te.te_cast_fp8_per_token(xt, E4)
    qwt, swt = te.te_cast_fp8_per_token(wt_, E4)
    yt = torch.empty((256, 256), dtype=torch.float32, device="cuda")
    ot = torch.zeros((256, 256), dtype=torch.float32, device="cuda")
    f = 2.0 * 256 * 256 * 512
    return {
        "tiny_fprop_bias_gelu_256x256x512": Case(
            lambda: te.te_fp8_gemm_fwd(qxt, sxt, E4, qwt, swt, E4, bias=bt, epilogue=te.TE_EPI_BIAS | te.TE_EPI_GELU,
                                       y=yt, y_dtype=te.TE_DTYPE_F32, accum=te.TE_ACCUM_FULL_FP32), f),
        "tiny_wgrad_256x256x512": Case(
            lambda: te.te_fp8_wgrad_accum(qxt, sxt, E4, qwt, swt, E4, ot, te.TE_ACCUM_FULL_FP32), f),
    }, []


def group_dense_wgrad(te, torch, g):
    """7168 x 2112 x 4096 weight gradient: FULL on IEEE-scaled operands (the headline kernel), FULL and
    FAST on power-of-two-scaled operands, the batched cast of both operands, and the step from
    token-major sources through the cast-transpose."""
    E4 = te.TE_DTYPE_E4M3
    T, M, N = 4096, 7168, 2112
    a, b = _randn(torch, g, (M, T), 1.0, 16), _randn(torch, g, (N, T), 1.0, 17)
    qa, sa = te.te_cast_fp8_per_token(a, E4)
    qb, sb = te.te_cast_fp8_per_token(b, E4)
    pa, psa = te.te_cast_fp8_per_token(a, E4, te.TE_CAST_POW2_SCALE)
    pb, psb = te.te_cast_fp8_per_token(b, E4, te.TE_CAST_POW2_SCALE)
    o = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    bg = torch.empty((M,), dtype=torch.float32, device="cuda")
    dyt, xt = _randn(torch, g, (T, M), 1.0, 11), _randn(torch, g, (T, N), 1.0, 12)
    qa2 = torch.empty((M, T), dtype=torch.uint8, device="cuda")
    sa2 = torch.empty((T // 128, te.scale_ld(M)), dtype=torch.float32, device="cuda")
    qb2 = torch.empty((N, T), dtype=torch.uint8, device="cuda")
    sb2 = torch.empty((T // 128, te.scale_ld(N)), dtype=torch.float32, device="cuda")

    def token_major():
        te.te_cast_fp8_per_token_transpose(dyt, E4, rowwise=False, qt=qa2, scales_t=sa2)
        te.te_cast_fp8_per_token_transpose(xt, E4, rowwise=False, qt=qb2, scales_t=sb2)
        te.te_fp8_wgrad_accum(qa2, sa2, E4, qb2, sb2, E4, o, te.TE_ACCUM_FULL_FP32)

    f = 2.0 * M * N * T
    cast_bytes = (M + N) * T * 3 + (M + N) * (T // 128) * 4
    return {
        "wgrad_full_7168x2112x4096": Case(lambda: te.te_fp8_wgrad_accum(qa, sa, E4, qb, sb, E4, o,
                                                                        te.TE_ACCUM_FULL_FP32), f),
        "wgrad_bgrad_full_7168x2112x4096": Case(
            lambda: te.te_fp8_wgrad_accum_bgrad(qa, sa, E4, qb, sb, E4, o, bg, te.TE_ACCUM_FULL_FP32), f,
            note="out += A B^T and the bias gradient as the row sums of A (dY^T) in the same call"),
        "wgrad_pow2_full_7168x2112x4096": Case(lambda: te.te_fp8_wgrad_accum(pa, psa, E4, pb, psb, E4, o,
                                                                             te.TE_ACCUM_FULL_FP32), f),
        "wgrad_pow2_fast_7168x2112x4096": Case(lambda: te.te_fp8_wgrad_accum(pa, psa, E4, pb, psb, E4, o,
                                                                             te.TE_ACCUM_FAST), f),
        "cast_batch_e4m3_7168x4096_2112x4096": Case(
            lambda: te.te_cast_fp8_per_token_batch([a, b], E4, qs=[qa, qb], scales=[sa, sb]), nbytes=cast_bytes),
        "wgrad_from_token_major_7168x2112x4096": Case(
            token_major, f, note="cast-transpose dY and X (tokens x features, bf16) + out += A B^T"),
    }, [("wgrad_pow2_full_7168x2112x4096", "wgrad_pow2_fast_7168x2112x4096"),
        ("wgrad_full_7168x2112x4096", "wgrad_bgrad_full_7168x2112x4096")]


def group_fprop(te, torch, g):
    """8192 x 14336 x 4096 forward, bf16 out: NONE vs bias+GELU (+aux) in both policies, FAST on IEEE
    scales (every tile falls back to FULL) and on power-of-two scales, the quantising store, and the
    casts of the activation."""
    E4 = te.TE_DTYPE_E4M3
    M, N, K = 8192, 14336, 4096
    x, w, b = _randn(torch, g, (M, K), 1.0, 1), _randn(torch, g, (N, K), 0.02, 2), _randn(torch, g, (N,), 0.1, 3)
    qx, sx = te.te_cast_fp8_per_token(x, E4)
    qw, sw = te.te_cast_fp8_per_token(w, E4)
    px, psx = te.te_cast_fp8_per_token(x, E4, te.TE_CAST_POW2_SCALE)
    pw, psw = te.te_cast_fp8_per_token(w, E4, te.TE_CAST_POW2_SCALE)
    y = _randn(torch, g, (M, N), 1.0, 9)       # (filled: the cast-transpose case reads it)
    z = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    qy = torch.empty((M, N), dtype=torch.uint8, device="cuda")
    qys = torch.empty((N // 128, te.scale_ld(M)), dtype=torch.float32, device="cuda")
    BG, BGA = te.TE_EPI_BIAS | te.TE_EPI_GELU, te.TE_EPI_BIAS | te.TE_EPI_GELU | te.TE_EPI_AUX_PREACT
    FULL, FAST = te.TE_ACCUM_FULL_FP32, te.TE_ACCUM_FAST
    f = 2.0 * M * N * K

    def fw(a, sa, bb, sb, epi, acc):
        return lambda: te.te_fp8_gemm_fwd(a, sa, E4, bb, sb, E4, bias=b if epi & te.TE_EPI_BIAS else None,
                                          epilogue=epi, y=y, preact=z if epi & te.TE_EPI_AUX_PREACT else None,
                                          accum=acc)

    qxt = torch.empty((K, M), dtype=torch.uint8, device="cuda")
    sxt = torch.empty((M // 128, te.scale_ld(K)), dtype=torch.float32, device="cuda")
    qyt = torch.empty((N, M), dtype=torch.uint8, device="cuda")
    qyts = torch.empty((M // 128, te.scale_ld(N)), dtype=torch.float32, device="cuda")
    cast_bytes = M * K * 3 + M * (K // 128) * 4
    ct_bytes = M * K * 2 + 2 * M * K + 2 * M * (K // 128) * 4
    cases = {
        "fprop_none_full": Case(fw(qx, sx, qw, sw, te.TE_EPI_NONE, FULL), f),
        "fprop_bias_gelu_full": Case(fw(qx, sx, qw, sw, BG, FULL), f),
        "fprop_none_fast": Case(fw(qx, sx, qw, sw, te.TE_EPI_NONE, FAST), f,
                                note="IEEE scales: every tile takes the FULL update"),
        "fprop_none_fast_pow2": Case(fw(px, psx, pw, psw, te.TE_EPI_NONE, FAST), f),
        "fprop_bias_gelu_fast_pow2": Case(fw(px, psx, pw, psw, BG, FAST), f),
        "fprop_bias_gelu_aux_fast_pow2": Case(fw(px, psx, pw, psw, BGA, FAST), f),
        "fprop_bias_gelu_aux_full": Case(fw(qx, sx, qw, sw, BGA, FULL), f),
        "fprop_bias_gelu_quant_e4m3_fast_pow2": Case(
            lambda: te.te_fp8_gemm_fwd_quant(px, psx, E4, pw, psw, E4, bias=b, epilogue=BG, q=qy, q_scales=qys,
                                             accum=FAST), f),
        "fprop_bias_gelu_aux_quant_both_e4m3_fast_pow2": Case(
            lambda: te.te_fp8_gemm_fwd_quant(px, psx, E4, pw, psw, E4, bias=b, epilogue=BGA, q=qy, q_scales=qys,
                                             preact=z, accum=FAST, transposed=True, qt=qyt, qt_scales=qyts), f,
            note="the fused forward of an MLP's first layer: pre-activation, and the cast of GELU's output "
                 "in both layouts"),
        "cast_and_transpose_e4m3_8192x14336": Case(
            lambda: te.te_cast_fp8_per_token_transpose(y, E4, q=qy, scales=qys, qt=qyt, scales_t=qyts),
            nbytes=M * N * 4 + 2 * M * (N // 128) * 4),
        "cast_e4m3_8192x4096": Case(lambda: te.te_cast_fp8_per_token(x, E4, q=qx, scales=sx), nbytes=cast_bytes),
        "cast_and_transpose_e4m3_8192x4096": Case(
            lambda: te.te_cast_fp8_per_token_transpose(x, E4, q=qx, scales=sx, qt=qxt, scales_t=sxt), nbytes=ct_bytes),
    }
    pairs = [("fprop_none_full", "fprop_bias_gelu_full"), ("fprop_none_full", "fprop_none_fast"),
             ("fprop_none_fast_pow2", "fprop_bias_gelu_fast_pow2"),
             ("fprop_none_fast_pow2", "fprop_bias_gelu_aux_fast_pow2"),
             ("fprop_bias_gelu_full", "fprop_bias_gelu_aux_full"),
             ("fprop_bias_gelu_fast_pow2", "fprop_bias_gelu_quant_e4m3_fast_pow2"),
             ("fprop_bias_gelu_aux_fast_pow2", "fprop_bias_gelu_aux_quant_both_e4m3_fast_pow2")]
    return cases, pairs


def group_dgrad(te, torch, g):
    """dX [8192 x 4096] = dY [8192 x 14336] (e5m2) W^T (e4m3); the gradient at the pre-activation shape
    [8192 x 14336] (contraction 4096) plain, with dGELU + bias-grad (atomic, deterministic, quantising
    to e5m2); the e5m2 cast of the gradient."""
    E4, E5 = te.TE_DTYPE_E4M3, te.TE_DTYPE_E5M2
    FULL, FAST = te.TE_ACCUM_FULL_FP32, te.TE_ACCUM_FAST
    M, N, K = 8192, 4096, 14336
    dy, wt = _randn(torch, g, (M, K), 1e-3, 4), _randn(torch, g, (N, K), 0.02, 5)
    qd, sd = te.te_cast_fp8_per_token(dy, E5)
    qt, st = te.te_cast_fp8_per_token(wt, E4)
    dx = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    f = 2.0 * M * N * K
    cast_bytes = M * K * 3 + M * (K // 128) * 4
    M2, N2, K2 = 8192, 14336, 4096
    do, w2t, zz = _randn(torch, g, (M2, K2), 1e-3, 6), _randn(torch, g, (N2, K2), 0.02, 7), \
        _randn(torch, g, (M2, N2), 1.28, 8)
    qo, so = te.te_cast_fp8_per_token(do, E5)
    q2, s2 = te.te_cast_fp8_per_token(w2t, E4)
    dz = _randn(torch, g, (M2, N2), 1e-3, 10)  # (filled: the cast-transpose case reads it)
    bg = torch.empty((N2,), dtype=torch.float32, device="cuda")
    ws = torch.empty((te.load_library().te_fp8_dgrad_bgrad_workspace_bytes(M2, N2),), dtype=torch.uint8,
                     device="cuda")
    qz = torch.empty((M2, N2), dtype=torch.uint8, device="cuda")
    qzs = torch.empty((N2 // 128, te.scale_ld(M2)), dtype=torch.float32, device="cuda")
    qzt = torch.empty((N2, M2), dtype=torch.uint8, device="cuda")
    qzts = torch.empty((M2 // 128, te.scale_ld(N2)), dtype=torch.float32, device="cuda")
    f2 = 2.0 * M2 * N2 * K2
    DB = te.TE_EPI_DGELU | te.TE_EPI_BGRAD
    cases = {
        "dgrad_dx_full": Case(lambda: te.te_fp8_gemm_dgrad(qd, sd, E5, qt, st, E4, dx=dx, accum=FULL), f),
        "dgrad_dx_fast": Case(lambda: te.te_fp8_gemm_dgrad(qd, sd, E5, qt, st, E4, dx=dx, accum=FAST), f,
                              note="IEEE scales: every tile takes the FULL update"),
        "cast_e5m2_8192x14336": Case(lambda: te.te_cast_fp8_per_token(dy, E5, q=qd, scales=sd), nbytes=cast_bytes),
        "dgrad_dz_none_full": Case(lambda: te.te_fp8_gemm_dgrad(qo, so, E5, q2, s2, E4, dx=dz, accum=FULL), f2),
        "dgrad_dz_dgelu_bgrad_full": Case(
            lambda: te.te_fp8_gemm_dgrad(qo, so, E5, q2, s2, E4, epilogue=DB, preact=zz, bias_grad=bg, dx=dz,
                                         accum=FULL), f2),
        "dgrad_dz_dgelu_bgrad_deterministic_full": Case(
            lambda: te.te_fp8_gemm_dgrad_deterministic(qo, so, E5, q2, s2, E4, bg, epilogue=DB, preact=zz,
                                                       workspace=ws, dx=dz, accum=FULL), f2),
        "dgrad_dz_dgelu_bgrad_quant_e5m2_full": Case(
            lambda: te.te_fp8_gemm_dgrad_quant(qo, so, E5, q2, s2, E4, epilogue=DB, preact=zz, bias_grad=bg, q=qz,
                                               q_scales=qzs, accum=FULL), f2),
        "dgrad_dz_dgelu_bgrad_quant_both_e5m2_full": Case(
            lambda: te.te_fp8_gemm_dgrad_quant(qo, so, E5, q2, s2, E4, epilogue=DB, preact=zz, bias_grad=bg, q=qz,
                                               q_scales=qzs, accum=FULL, transposed=True, qt=qzt, qt_scales=qzts),
            f2, note="the data gradient at an MLP's hidden layer, cast in both layouts (the next data and "
                     "weight gradients' operands)"),
        "cast_and_transpose_e5m2_8192x14336": Case(
            lambda: te.te_cast_fp8_per_token_transpose(dz, E5, q=qz, scales=qzs, qt=qzt, scales_t=qzts),
            nbytes=M2 * N2 * 4 + 2 * M2 * (N2 // 128) * 4),
    }
    pairs = [("dgrad_dz_none_full", "dgrad_dz_dgelu_bgrad_full"),
             ("dgrad_dz_none_full", "dgrad_dz_dgelu_bgrad_deterministic_full"),
             ("dgrad_dz_dgelu_bgrad_full", "dgrad_dz_dgelu_bgrad_quant_e5m2_full"),
             ("dgrad_dz_dgelu_bgrad_full", "dgrad_dz_dgelu_bgrad_quant_both_e5m2_full")]
    return cases, pairs


def group_kgrouped(te, torch, g):
    """8 experts, 2048 x 7168, per-expert K multinomial in blocks of 128 summing to 32768, FULL; the
    group sizes on the host and on the device."""
    import workloads as W
    E4 = te.TE_DTYPE_E4M3
    G, M, N, S = 8, 2048, 7168, 32768
    gk = W.moe_group_k(np.random.SeedSequence(5).spawn(4)[2], G, S).tolist()
    a, bm = _randn(torch, g, (M, S), 1.0, 9), _randn(torch, g, (N, S), 1.0, 10)
    qa, sa = te.te_cast_fp8_per_token(a, E4)
    qb, sb = te.te_cast_fp8_per_token(bm, E4)
    del a, bm
    o = torch.zeros((G, M, N), dtype=torch.float32, device="cuda")
    gk_dev = torch.tensor(gk, dtype=torch.int64, device="cuda")
    f = 2.0 * M * N * S
    return {
        "kgrouped_wgrad_full": Case(lambda: te.te_fp8_kgrouped_wgrad(qa, sa, E4, qb, sb, E4, gk, o,
                                                                     te.TE_ACCUM_FULL_FP32), f, note=str(gk)),
        "kgrouped_wgrad_device_sizes_full": Case(
            lambda: te.te_fp8_kgrouped_wgrad_device_sizes(qa, sa, E4, qb, sb, E4, gk_dev, o, te.TE_ACCUM_FULL_FP32), f),
    }, []


def group_mgrouped(te, torch, g):
    """M-grouped expert forward: 8 experts x 1024 tokens (4 blocks of 256 rows each), N = 4096,
    K = 7168, bias + GELU, bf16 out."""
    E4 = te.TE_DTYPE_E4M3
    G, T, N, K = 8, 8192, 4096, 7168
    xg, wg, bgs = _randn(torch, g, (T, K), 1.0, 13), _randn(torch, g, (G * N, K), 0.02, 14), \
        _randn(torch, g, (G, N), 0.1, 15)
    qx, sx = te.te_cast_fp8_per_token(xg, E4)
    qw, sw = te.te_cast_fp8_per_token(wg, E4)
    qw = qw.view(G, N, K)
    # per-expert scale arrays in the [G][K/128][scale_ld(N)] layout (N is a multiple of 4)
    sw = sw.view(K // 128, G, N).permute(1, 0, 2).contiguous()
    blocks = torch.arange(T // 256, device="cuda", dtype=torch.int32) // ((T // 256) // G)
    yg = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    # the experts' data gradient at the hidden layer: dZ [T, 7168] = dO [T, 4096] W2[e]^T, dGELU on the
    # saved pre-activation, per-expert bias gradients (atomic and deterministic)
    E5 = te.TE_DTYPE_E5M2
    F = K
    qdo, sdo = te.te_cast_fp8_per_token(_randn(torch, g, (T, N), 1e-3, 16), E5)
    qw2, sw2 = te.te_cast_fp8_per_token(_randn(torch, g, (G * F, N), 0.02, 17), te.TE_DTYPE_E4M3)
    qw2 = qw2.view(G, F, N)
    sw2 = sw2.view(N // 128, G, F).permute(1, 0, 2).contiguous()
    zg = _randn(torch, g, (T, F), 1.28, 18)
    dzg = torch.empty((T, F), dtype=torch.bfloat16, device="cuda")
    bgg = torch.empty((G * F,), dtype=torch.float32, device="cuda")
    wsg = torch.empty((te.load_library().te_fp8_dgrad_bgrad_workspace_bytes(T, F),), dtype=torch.uint8, device="cuda")
    DB = te.TE_EPI_DGELU | te.TE_EPI_BGRAD
    fd = 2.0 * T * F * N
    return {
        "mgrouped_fwd_bias_gelu_full_8x1024x4096x7168": Case(
            lambda: te.te_fp8_mgrouped_gemm_fwd(qx, sx, E4, qw, sw, E4, blocks, bias=bgs,
                                                epilogue=te.TE_EPI_BIAS | te.TE_EPI_GELU, y=yg,
                                                accum=te.TE_ACCUM_FULL_FP32), 2.0 * T * N * K),
        "mgrouped_dgrad_dgelu_bgrad_full_8x1024x7168x4096": Case(
            lambda: te.te_fp8_mgrouped_gemm_dgrad(qdo, sdo, E5, qw2, sw2, te.TE_DTYPE_E4M3, blocks, epilogue=DB,
                                                  preact=zg, bias_grad=bgg, dx=dzg, accum=te.TE_ACCUM_FULL_FP32), fd),
        "mgrouped_dgrad_dgelu_bgrad_deterministic_full_8x1024x7168x4096": Case(
            lambda: te.te_fp8_mgrouped_gemm_dgrad_deterministic(qdo, sdo, E5, qw2, sw2, te.TE_DTYPE_E4M3, blocks, bgg,
                                                                epilogue=DB, preact=zg, workspace=wsg, dx=dzg,
                                                                accum=te.TE_ACCUM_FULL_FP32), fd),
    }, [("mgrouped_dgrad_dgelu_bgrad_full_8x1024x7168x4096",
         "mgrouped_dgrad_dgelu_bgrad_deterministic_full_8x1024x7168x4096")]


def group_modules(te, torch, g):
    """One training step (forward + backward) of the library's MLP block, fc1 4096 -> 14336, GELU,
    fc2 14336 -> 4096, on 8192 tokens: every GEMM, cast and epilogue is a library call (the modules
    add autograd's bookkeeping); the fp8 weights come from the cache."""
    from fp8_linear_layer_amd import linear as lin
    T, D, H = 8192, 4096, 14336
    gen = torch.Generator(device="cuda").manual_seed(19)
    m = lin.Fp8Mlp(D, H, D, generator=gen)
    mp = lin.Fp8Mlp(D, H, D, generator=torch.Generator(device="cuda").manual_seed(19), pow2_scales=True)
    x = _randn(torch, g, (T, D), 1.0, 20).requires_grad_(True)
    dy = _randn(torch, g, (T, D), 1e-3, 21)

    def step(mod):
        mod(x).backward(dy)
        x.grad = None
        mod.b1.grad = None
        mod.b2.grad = None
    f = 6 * 2.0 * T * D * H
    return {"mlp_step_8192x4096x14336": Case(lambda: step(m), f,
                                              note="forward (2 GEMMs) + backward (4 GEMMs) + casts"),
            "mlp_step_pow2_8192x4096x14336": Case(
                lambda: step(mp), f, note="the same with pow2_scales: x, h and the weights cast with power-of-two "
                                          "scales, both forward GEMMs on FAST (chained)")}, \
        [("mlp_step_8192x4096x14336", "mlp_step_pow2_8192x4096x14336")]


GROUPS = [group_tiny, group_dense_wgrad, group_fprop, group_dgrad, group_kgrouped, group_mgrouped, group_modules]
# the cases of each group (so that --case sets up only its own group's inputs)
GROUP_CASES = {
    group_tiny: ("tiny_fprop_bias_gelu_256x256x512", "tiny_wgrad_256x256x512"),
    group_dense_wgrad: ("wgrad_full_7168x2112x4096", "wgrad_bgrad_full_7168x2112x4096", "wgrad_pow2_full_7168x2112x4096",
                        "wgrad_pow2_fast_7168x2112x4096",
                        "cast_batch_e4m3_7168x4096_2112x4096", "wgrad_from_token_major_7168x2112x4096"),
    group_fprop: ("fprop_none_full", "fprop_bias_gelu_full", "fprop_none_fast", "fprop_none_fast_pow2",
                  "fprop_bias_gelu_fast_pow2", "fprop_bias_gelu_aux_fast_pow2", "fprop_bias_gelu_aux_full",
                  "fprop_bias_gelu_quant_e4m3_fast_pow2",
                  "fprop_bias_gelu_aux_quant_both_e4m3_fast_pow2", "cast_and_transpose_e4m3_8192x14336",
                  "cast_e4m3_8192x4096", "cast_and_transpose_e4m3_8192x4096"),
    group_dgrad: ("dgrad_dx_full", "dgrad_dx_fast", "cast_e5m2_8192x14336", "dgrad_dz_none_full",
                  "dgrad_dz_dgelu_bgrad_full", "dgrad_dz_dgelu_bgrad_deterministic_full",
                  "dgrad_dz_dgelu_bgrad_quant_e5m2_full", "dgrad_dz_dgelu_bgrad_quant_both_e5m2_full",
                  "cast_and_transpose_e5m2_8192x14336"),
    group_kgrouped: ("kgrouped_wgrad_full", "kgrouped_wgrad_device_sizes_full"),
    group_mgrouped: ("mgrouped_fwd_bias_gelu_full_8x1024x4096x7168", "mgrouped_dgrad_dgelu_bgrad_full_8x1024x7168x4096",
                     "mgrouped_dgrad_dgelu_bgrad_deterministic_full_8x1024x7168x4096"),
    group_modules: ("mlp_step_8192x4096x14336", "mlp_step_pow2_8192x4096x14336"),
}


def _summ(case, times):
    t = np.asarray(times)
    med = float(np.median(t))
    rec = {"ms": round(med, 5), "p10_ms": round(float(np.percentile(t, 10)), 5),
           "p90_ms": round(float(np.percentile(t, 90)), 5), "rounds": int(t.size)}
    if case.flop:
        rec["tflops"] = round(case.flop / med / 1e9, 1)
        rec["frac_fp8_peak"] = round(case.flop / med / 1e9 / MFMA_FP8_PEAK_TFLOPS, 4)
    if case.nbytes:
        rec["gbs"] = round(case.nbytes / med / 1e6, 1)
        rec["frac_hbm"] = round(case.nbytes / med / 1e6 / HBM_PEAK_GBS, 4)
    if case.note:
        rec["note"] = case.note
    return rec


def breakdown(te, torch, rounds=20, reps=10):
    """Every other workload's kernel time.  Within a group the cases are timed interleaved (each round
    times every case once, `reps` back-to-back launches each), after a common warm-up; the median and
    the 10th/90th percentiles over the rounds are reported, and each epilogue's overhead is the median
    over rounds of its time divided by its base case's time in the same round."""
    g = torch.Generator(device="cuda")
    out = {}
    for grp in GROUPS:
        cases, pairs = grp(te, torch, g)
        # settle the clocks on this group's first case before the measured rounds
        first = next(iter(cases.values())).fn
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.3:
            for _ in range(10):
                first()
            torch.cuda.synchronize()
        n = reps if not grp.__name__.endswith("tiny") else 50
        times = timed_interleaved({k: c.fn for k, c in cases.items()}, n, rounds)
        for k, c in cases.items():
            out[k] = _summ(c, times[k])
            if k.startswith("tiny"):
                out[k]["us"] = round(out[k]["ms"] * 1e3, 2)
        for base, epi in pairs:
            r = np.asarray(times[epi]) / np.asarray(times[base])
            out[epi].setdefault("overhead_vs", {})[base] = {
                "median": round(float(np.median(r)) - 1.0, 4),
                "p10": round(float(np.percentile(r, 10)) - 1.0, 4),
                "p90": round(float(np.percentile(r, 90)) - 1.0, 4)}
        del cases
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def run_case(te, torch, name, reps, warm):
    """One case alone, `warm` + `reps` launches (the command the committed rocprofv3 summaries run)."""
    g = torch.Generator(device="cuda")
    for grp in GROUPS:
        if name not in GROUP_CASES[grp]:
            continue
        cases, _ = grp(te, torch, g)
        if name in cases:
            c = cases[name]
            for _ in range(warm):
                c.fn()
            torch.cuda.synchronize()
            # (back-to-back launches between one event pair, as in the breakdown)
            per = min(10, reps)
            times = timed_interleaved({name: c.fn}, per, max(1, reps // per), warm=0)
            rec = {"case": name, **_summ(c, times[name])}
            print(json.dumps(rec), flush=True)
            return
        del cases
    raise SystemExit(f"unknown case {name!r}")


def cpu_baseline(rows: int, min_seconds: float):
    """The oracle (as it stands) on a bounded sample of the same step: cast `rows` rows of
    A and all of B, then `rows` x N outputs of the wgrad product, repeated until
    `min_seconds` of CPU work have run; scaled to TFLOP/s."""
    import oracle
    import workloads as W
    M, N, K = 7168, 2112, 4096
    rows = max(1, min(rows, M))
    s = np.random.SeedSequence(2).spawn(3)
    a = W.normal_bf16(s[0], (M, K))[:rows]
    b = W.normal_bf16(s[1], (N, K))
    out0 = W.normal_f32(s[2], (M, N))[:rows]
    runs, t0 = 0, time.perf_counter()
    while True:
        qa, sa = oracle.cast_per_token(a, oracle.E4M3)
        qb, sb = oracle.cast_per_token(b, oracle.E4M3)
        o, d = oracle.gemm_nt(qa, sa, oracle.E4M3, qb, sb, oracle.E4M3)
        oracle.wgrad(o, d, out0)
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    flop = 2.0 * rows * N * K * runs
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{rows} of 7168 output rows (all 2112 columns, K=4096) incl. the cast of those rows and of B, "
                      f"{runs} run(s) in {dt:.1f} s"}


def ref_copy(torch):
    """Three plain 1 GiB device copies: the reference reading of the HBM byte counters."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only (the library has no multi-GPU path); --gpus must be 1"}))
        sys.exit(2)
    import torch
    import fp8_linear_layer_amd as te
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    te.load_library()
    torch.cuda.set_device(0)
    if args.case:
        if args.ref_copy:
            ref_copy(torch)
        run_case(te, torch, args.case, args.reps, args.warmup)
        return
    M, N, K = 7168, 2112, 4096
    inp = W.dense_wgrad_inputs()
    a = torch.from_numpy(inp["a"]).cuda().view(torch.bfloat16)
    b = torch.from_numpy(inp["b"]).cuda().view(torch.bfloat16)
    out = torch.from_numpy(inp["out0"]).cuda()
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((K // 128, te.scale_ld(M)), dtype=torch.float32, device="cuda")
    qb = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sb = torch.empty((K // 128, te.scale_ld(N)), dtype=torch.float32, device="cuda")
    E4 = te.TE_DTYPE_E4M3
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]

    def step(i=None):
        # both operands cast in one launch (te_cast_fp8_per_token_batch)
        te.te_cast_fp8_per_token_batch([a, b], E4, qs=[qa, qb], scales=[sa, sb])
        if i is not None:
            ev[i][0].record(stream)
        te.te_fp8_wgrad_accum(qa, sa, E4, qb, sb, E4, out, te.TE_ACCUM_FULL_FP32)
        if i is not None:
            ev[i][1].record(stream)

    def cast_only():
        te.te_cast_fp8_per_token_batch([a, b], E4, qs=[qa, qb], scales=[sa, sb])

    if args.ref_copy:
        ref_copy(torch)
    # (the garbage collector is paused over the warm-up and timed steps, as
    # timeit does: a collection pass mid-loop leaves the GPU idle for ms)
    gc.collect()
    gc.disable()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    gc.enable()
    ms_step = total * 1e3 / args.steps
    # (after the timed region) the GEMM's time inside a step, event pair
    # around its launch: includes the dispatch gap in front of it
    for i in range(len(ev)):
        step(i)
    torch.cuda.synchronize()
    in_step_ms = float(np.mean([s.elapsed_time(e) for s, e in ev]))
    cast_ms, _ = timed(cast_only, args.kernel_reps)
    # Cold-cache step (secondary): before each step a 512 MiB fill evicts the
    # 256 MB Infinity Cache and the L2s; an event pair on the stream brackets
    # the step alone (it includes the dispatch gap after the fill).
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = []
    for i in range(args.cold_steps + 2):
        flush.fill_(i & 0xFF)
        cs, ce = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cs.record(stream)
        step()
        ce.record(stream)
        ce.synchronize()
        if i >= 2:
            cold.append(cs.elapsed_time(ce))
    del flush
    cold_ms = float(np.median(cold))
    # The kernel's own duration: back-to-back launches between one event pair
    # on the launch stream (an event pair around a single launch also counts
    # the dispatch gap in front of it): after 100 launches that bring the clock
    # back up from the cache-flush loop, the median of 10 rounds of
    # kernel_reps back-to-back launches, one event pair each.
    gemm_ms, _ = timed(lambda: te.te_fp8_wgrad_accum(qa, sa, E4, qb, sb, E4, out, te.TE_ACCUM_FULL_FP32),
                       args.kernel_reps, warm=100, rounds=10)
    flop = 2.0 * M * N * K
    value = flop / (ms_step * 1e-3) / 1e12
    achieved = flop / (gemm_ms * 1e-3) / 1e12
    traffic = traffic_from_profile("wgrad_full_7168x2112x4096")
    rec = {
        "metric": "FP8 GEMM TFLOPS (fprop/dgrad/wgrad) and % of MI355X FP8 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / PAGES_TFLOPS_SAME_SHAPE, 4),
        "dtype": "e4m3",
        "data": "synthetic",
        "config": {"workload": "dense-wgrad-7168x2112x4096", "M": M, "N": N, "K": K,
                   "step": "cast A + cast B in one launch (bf16 -> e4m3, 1x128 fp32 scales) + out += A B^T (fp32)",
                   "accum": "full_fp32", "frac_of_fp8_peak": round(value / MFMA_FP8_PEAK_TFLOPS, 4),
                   "cold_cache": {"ms_per_step": round(cold_ms, 5), "tflops": round(flop / (cold_ms * 1e-3) / 1e12, 2),
                                  "note": "median of steps each after a 512 MiB fill (caches evicted); secondary"}},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_FP8_PEAK_TFLOPS, 4), "traffic": traffic,
                     "kernel": "gemm_nt_kernel (wgrad, full)", "kernel_ms": round(gemm_ms, 5),
                     "kernel_ms_in_step": round(in_step_ms, 5),
                     "casts_ms": round(cast_ms, 5)},
    }
    if not args.no_breakdown:
        rec["breakdown"] = breakdown(te, torch, rounds=args.breakdown_rounds)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(args.cpu_rows, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
