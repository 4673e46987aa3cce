"""Host-side checks of the C ABI (CPU only, no GPU calls).

The library validates every argument on the host before anything is
enqueued, so each rejected call here returns its status without touching HIP.
Pointers are dummies (aligned or deliberately misaligned addresses that are
never dereferenced).
"""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "te_fp8.h")

te = pytest.importorskip("fp8_linear_layer_amd")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(te.LIB_PATH):
        pytest.skip("libte_fp8.so not built")
    return te.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(te_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_five_operations():
    fns = header_functions()
    for name in ("te_cast_fp8_per_token", "te_fp8_gemm_fwd", "te_fp8_gemm_dgrad",
                 "te_fp8_wgrad_accum", "te_fp8_kgrouped_wgrad"):
        assert name in fns


def test_library_exports_every_declared_symbol(lib):
    fns = header_functions()
    assert fns, "no declarations parsed"
    missing = [f for f in fns if not hasattr(lib, f)]
    assert not missing, missing
    assert set(te.EXPORTED) <= set(fns)


A = 0x10000          # 16-byte aligned dummy device addresses, never dereferenced
B = 0x20000
S = 0x30000
O = 0x40000
BIAS = 0x50000
Z = 0x60000
MIS = 0x10008        # 8-byte but not 16-byte aligned

INV, MISAL = 1, 2


def p(x):
    return ctypes.c_void_p(x) if x else None


def wgrad(lib, a=A, sa=S, da=1, b=B, sb=S, db=1, M=256, N=256, K=512, out=O, ld=256, accum=1):
    return lib.te_fp8_wgrad_accum(p(a), p(sa), da, p(b), p(sb), db, M, N, K, p(out), ld, accum, None)


@pytest.mark.parametrize("kw,status", [
    (dict(a=0), INV), (dict(sb=0), INV), (dict(out=0), INV),
    (dict(M=0), INV), (dict(N=-3), INV), (dict(K=0), INV), (dict(K=100), INV), (dict(K=200), INV),
    (dict(K=(1 << 22) + 128), INV),
    (dict(da=3), INV), (dict(db=4), INV), (dict(da=0), INV),
    (dict(accum=0), INV), (dict(accum=3), INV),
    (dict(ld=255), INV), (dict(ld=258), MISAL),
    (dict(a=MIS), MISAL), (dict(b=MIS), MISAL), (dict(out=MIS), MISAL), (dict(sa=S + 2), MISAL),
    (dict(sa=S + 4), MISAL), (dict(sb=S + 8), MISAL),   # block-major scales are copied 16 bytes at a time
])
def test_wgrad_rejects(lib, kw, status):
    assert wgrad(lib, **kw) == status
    assert lib.te_last_error_message().decode()


def fwd(lib, bias=None, epi=0, y=O, ydt=3, ld=256, pre=None, ldp=0, accum=2, N=256):
    return lib.te_fp8_gemm_fwd(p(A), p(S), 1, p(B), p(S), 1, 256, N, 512, p(bias), epi,
                               p(y), ydt, ld, p(pre), ldp, accum, None)


@pytest.mark.parametrize("kw,status", [
    (dict(epi=1), INV),                         # BIAS without a bias pointer
    (dict(bias=BIAS), INV),                     # bias pointer without BIAS
    (dict(epi=4 | 2, pre=None), INV),           # AUX without preact
    (dict(epi=4, pre=Z, ldp=256), INV),         # AUX without GELU
    (dict(epi=8), INV), (dict(epi=16), INV),    # dgrad flags on the forward call
    (dict(pre=Z, ldp=256), INV),                # preact without AUX
    (dict(ydt=1), INV), (dict(ydt=0), INV),     # y must be bf16 or fp32
    (dict(ld=252, ydt=3), INV),                 # ld below N
    (dict(ld=260, ydt=3), MISAL),               # bf16 rows must be 16-byte multiples
    (dict(epi=1, bias=BIAS + 2), MISAL),
    (dict(epi=2 | 4, pre=Z, ldp=100), INV),
    (dict(y=MIS), MISAL),
])
def test_fwd_rejects(lib, kw, status):
    assert fwd(lib, **kw) == status


def dgrad(lib, epi=0, pre=None, ldp=0, bg=None, dx=O, dxdt=3, ld=256, accum=1):
    return lib.te_fp8_gemm_dgrad(p(A), p(S), 2, p(B), p(S), 1, 256, 256, 512, epi, p(pre), ldp, p(bg),
                                 p(dx), dxdt, ld, accum, None)


@pytest.mark.parametrize("kw,status", [
    (dict(epi=8), INV),                         # DGELU without preact
    (dict(epi=16), INV),                        # BGRAD without bias_grad
    (dict(pre=Z, ldp=256), INV),                # preact without DGELU
    (dict(bg=O + 4096), INV),                   # bias_grad without BGRAD
    (dict(epi=1), INV), (dict(epi=2), INV),     # forward flags on dgrad
    (dict(epi=8, pre=Z, ldp=128), INV),         # ld_preact below N
    (dict(epi=8, pre=Z + 8, ldp=256), MISAL),
    (dict(epi=16, bg=O + 4098), MISAL),
    (dict(dxdt=2), INV),
])
def test_dgrad_rejects(lib, kw, status):
    assert dgrad(lib, **kw) == status


def kgrouped(lib, gk, G=None, out=O, accum=1, M=256, N=256):
    arr = (ctypes.c_int64 * max(1, len(gk)))(*gk)
    G = len(gk) if G is None else G
    return lib.te_fp8_kgrouped_wgrad(p(A), p(S), 1, p(B), p(S), 1, M, N, ctypes.cast(arr, ctypes.c_void_p), G,
                                     p(out), accum, None)


@pytest.mark.parametrize("gk,G,status", [
    ([128, 100], None, INV), ([128, -128], None, INV), ([0, 0], None, INV), ([128], 0, INV),
    ([128] * 4, 1025, INV),
])
def test_kgrouped_rejects(lib, gk, G, status):
    assert kgrouped(lib, gk, G) == status


def test_kgrouped_null_group_k(lib):
    assert lib.te_fp8_kgrouped_wgrad(p(A), p(S), 1, p(B), p(S), 1, 256, 256, None, 2, p(O), 1, None) == INV


GK = 0x90000  # dummy device address of the group sizes


def kgrouped_dev(lib, gk=GK, G=4, sum_k=512, M=256, N=256, out=O, accum=1):
    return lib.te_fp8_kgrouped_wgrad_device_sizes(p(A), p(S), 1, p(B), p(S), 1, M, N, sum_k, p(gk), G, p(out),
                                                  accum, None)


QS = 0xB0000


QT, QTS = B + 0x200000, QS + 0x10000


def fwdq(lib, M=256, N=256, K=256, bias=0, epi=0, qdt=1, cf=0, q=B + 0x100000, ldq=256, qs=QS, qt=0, ldqt=0, qts=0,
         pre=0, ldpre=0, accum=2):
    return lib.te_fp8_gemm_fwd_quant(p(A), p(S), 1, p(B), p(S), 1, M, N, K, p(bias), epi, qdt, cf, p(q), ldq, p(qs),
                                     p(qt), ldqt, p(qts), p(pre), ldpre, accum, None)


# the transposed output: invalid alone or beside a valid row-wise one
QT_BAD = [
    (dict(q=0, qs=0), INV), (dict(q=0, qs=0, qt=QT, ldqt=256), INV), (dict(qt=QT, ldqt=256), INV),
    (dict(qts=QTS), INV), (dict(qt=QT, ldqt=256, qts=QTS, M=200), INV), (dict(qt=QT, ldqt=128, qts=QTS), INV),
    (dict(qt=QT + 8, ldqt=256, qts=QTS), MISAL), (dict(qt=QT, ldqt=264, qts=QTS), MISAL),
    (dict(qt=QT, ldqt=256, qts=QTS + 4), MISAL), (dict(q=0, qs=0, qt=QT, ldqt=256, qts=QTS, M=384), INV),
]


@pytest.mark.parametrize("kw,status", [
    (dict(N=200, ldq=208), INV), (dict(N=0), INV), (dict(epi=8), INV), (dict(epi=4), INV), (dict(epi=1), INV),
    (dict(bias=BIAS), INV), (dict(qdt=3), INV), (dict(cf=2), INV), (dict(q=0), INV), (dict(qs=0), INV),
    (dict(ldq=128), INV), (dict(q=MIS), MISAL), (dict(ldq=264), MISAL), (dict(qs=QS + 4), MISAL),
    (dict(pre=Z, ldpre=256), INV), (dict(epi=6), INV), (dict(accum=0), INV), (dict(K=64), INV),
] + QT_BAD)
def test_fwd_quant_rejects(lib, kw, status):
    assert fwdq(lib, **kw) == status


def dgq(lib, M=256, N=256, K=256, epi=0, pre=0, ldpre=0, bg=0, qdt=2, cf=0, q=B + 0x100000, ldq=256, qs=QS,
        qt=0, ldqt=0, qts=0, accum=1):
    return lib.te_fp8_gemm_dgrad_quant(p(A), p(S), 2, p(B), p(S), 1, M, N, K, epi, p(pre), ldpre, p(bg), qdt, cf,
                                       p(q), ldq, p(qs), p(qt), ldqt, p(qts), accum, None)


@pytest.mark.parametrize("kw,status", [
    (dict(N=200, ldq=208), INV), (dict(epi=1), INV), (dict(epi=8), INV), (dict(epi=16), INV), (dict(pre=Z), INV),
    (dict(bg=O), INV), (dict(epi=8, pre=Z, ldpre=128), INV), (dict(epi=8, pre=Z + 8, ldpre=256), MISAL),
    (dict(epi=16, bg=O + 2), MISAL), (dict(qdt=3), INV), (dict(cf=2), INV), (dict(q=0), INV), (dict(qs=0), INV),
    (dict(ldq=128), INV), (dict(q=MIS), MISAL), (dict(ldq=264), MISAL), (dict(qs=QS + 4), MISAL), (dict(accum=3), INV),
] + QT_BAD)
def test_dgrad_quant_rejects(lib, kw, status):
    assert dgq(lib, **kw) == status


WS = 0xC0000


@pytest.mark.parametrize("M,N,want", [(0, 5, 0), (5, 0, 0), (1, 1, 4 * 4 * 4), (256, 14336, 4 * 14336 * 4),
                                      (257, 14337, 8 * 14340 * 4), (8192, 14336, 128 * 14336 * 4)])
def test_dgrad_bgrad_workspace_bytes(lib, M, N, want):
    assert lib.te_fp8_dgrad_bgrad_workspace_bytes(M, N) == want


def dgd(lib, M=256, N=256, K=256, epi=16, pre=0, ldpre=0, bg=O, ws=WS, wsb=1 << 20, dx=Z, ldx=256, accum=1):
    return lib.te_fp8_gemm_dgrad_deterministic(p(A), p(S), 2, p(B), p(S), 1, M, N, K, epi, p(pre), ldpre, p(bg), p(ws),
                                               wsb, p(dx), 3, ldx, accum, None)


@pytest.mark.parametrize("kw,status", [
    (dict(epi=0), INV), (dict(epi=8, pre=Z + 0x1000, ldpre=256), INV), (dict(ws=0), INV), (dict(ws=WS + 8), MISAL),
    (dict(wsb=4 * 256 * 4 - 1), INV), (dict(bg=0), INV), (dict(bg=O + 2), MISAL), (dict(pre=Z + 0x1000), INV),
    (dict(epi=24, pre=0), INV), (dict(dx=0), INV), (dict(ldx=128), INV), (dict(K=100), INV), (dict(accum=0), INV),
])
def test_dgrad_deterministic_rejects(lib, kw, status):
    assert dgd(lib, **kw) == status


def wgrad_bg(lib, a=A, sa=S, da=1, b=B, sb=S, db=1, M=256, N=256, K=256, out=O, ld=256, bg=Z, accum=1):
    return lib.te_fp8_wgrad_accum_bgrad(p(a), p(sa), da, p(b), p(sb), db, M, N, K, p(out), ld, p(bg), accum, None)


@pytest.mark.parametrize("kw,status", [
    (dict(bg=0), INV), (dict(bg=Z + 2), MISAL), (dict(K=100), INV), (dict(K=0), INV), (dict(ld=100), INV),
    (dict(ld=258), MISAL), (dict(a=0), INV), (dict(b=0), INV), (dict(sa=0), INV), (dict(out=0), INV),
    (dict(M=0), INV), (dict(N=-1), INV), (dict(da=5), INV), (dict(accum=0), INV), (dict(accum=7), INV),
    (dict(a=MIS), MISAL), (dict(out=MIS), MISAL), (dict(sb=S + 4), MISAL), (dict(K=(1 << 22) + 128), INV),
])
def test_wgrad_bgrad_rejects(lib, kw, status):
    assert wgrad_bg(lib, **kw) == status
    assert "te_fp8_wgrad_accum_bgrad" in lib.te_last_error_message().decode()


def dgn(lib, M=512, N=256, K=256, epi=24, pre=Z, ldpre=256, bg=O, dx=0x70000, ldx=256, accum=1):
    return lib.te_fp8_gemm_dgrad_deterministic_noalloc(p(A), p(S), 2, p(B), p(S), 1, M, N, K, epi, p(pre), ldpre,
                                                       p(bg), p(dx), 3, ldx, accum, None)


@pytest.mark.parametrize("kw,status", [
    (dict(epi=8), INV), (dict(bg=0), INV), (dict(bg=O + 2), MISAL), (dict(pre=0), INV), (dict(dx=0), INV),
    (dict(ldx=128), INV), (dict(K=100), INV), (dict(accum=0), INV), (dict(ldpre=100), INV),
    # outputs whose column sums exceed the 8 MiB static scratch
    (dict(M=8192, N=16388, ldpre=16392, ldx=16392), INV), (dict(M=1 << 20, N=256), INV),
])
def test_dgrad_noalloc_rejects(lib, kw, status):
    assert dgn(lib, **kw) == status
    assert "te_fp8_gemm_dgrad_deterministic_noalloc" in lib.te_last_error_message().decode()


def test_dgrad_noalloc_limit_is_the_header_constant(lib):
    text = open(HEADER).read()
    assert "#define TE_NOALLOC_SCRATCH_BYTES (8 << 20)" in text
    assert te.NOALLOC_SCRATCH_BYTES == 8 << 20
    assert lib.te_fp8_dgrad_bgrad_workspace_bytes(8192, 16384) <= te.NOALLOC_SCRATCH_BYTES


MB = 0xA0000  # dummy device address of the per-block experts


def mgrouped(lib, mb=MB, G=4, sum_m=512, N=256, K=256, bias=0, epi=0, y=O, ydt=4, ldy=256, pre=0, ldpre=0, accum=2):
    return lib.te_fp8_mgrouped_gemm_fwd(p(A), p(S), 1, p(B), p(S), 1, sum_m, N, K, G, p(mb), p(bias), epi, p(y), ydt,
                                        ldy, p(pre), ldpre, accum, None)


def mgrouped_dg(lib, mb=MB, G=4, sum_m=512, N=256, K=256, epi=16, pre=0, ldpre=0, bg=O, dx=Z, dxdt=3, ldx=256,
                accum=1):
    return lib.te_fp8_mgrouped_gemm_dgrad(p(A), p(S), 2, p(B), p(S), 1, sum_m, N, K, G, p(mb), epi, p(pre), ldpre,
                                          p(bg), p(dx), dxdt, ldx, accum, None)


@pytest.mark.parametrize("kw,status", [
    (dict(mb=0), INV), (dict(mb=MB + 2), MISAL), (dict(G=0), INV), (dict(G=1025), INV), (dict(sum_m=300), INV),
    (dict(epi=1), INV), (dict(epi=8), INV), (dict(epi=24, pre=Z + 0x10000, ldpre=128), INV),
    (dict(epi=24, pre=Z + 0x10008, ldpre=256), MISAL), (dict(bg=0), INV), (dict(epi=0), INV),
    (dict(bg=O + 2), MISAL), (dict(dx=0), INV), (dict(ldx=128), INV), (dict(accum=0), INV),
])
def test_mgrouped_dgrad_rejects(lib, kw, status):
    assert mgrouped_dg(lib, **kw) == status


WSM = 0xB0000  # dummy device address of the M-grouped column-sum workspace


def mgrouped_dgd(lib, mb=MB, G=4, sum_m=512, N=256, K=256, epi=16, pre=0, ldpre=0, bg=O, ws=WSM, wsb=1 << 20, dx=Z,
                 dxdt=3, ldx=256, accum=1):
    return lib.te_fp8_mgrouped_gemm_dgrad_deterministic(p(A), p(S), 2, p(B), p(S), 1, sum_m, N, K, G, p(mb), epi,
                                                        p(pre), ldpre, p(bg), p(ws), wsb, p(dx), dxdt, ldx, accum,
                                                        None)


@pytest.mark.parametrize("kw,status", [
    (dict(ws=0), INV), (dict(ws=WSM + 8), MISAL), (dict(wsb=8 * 256 * 4 - 4), INV), (dict(epi=0), INV),
    (dict(epi=8), INV), (dict(bg=0), INV), (dict(bg=O + 2), MISAL), (dict(mb=0), INV), (dict(G=0), INV),
    (dict(sum_m=300), INV), (dict(dx=0), INV), (dict(ldx=128), INV), (dict(accum=0), INV),
    (dict(epi=24, pre=0), INV),
])
def test_mgrouped_dgrad_deterministic_rejects(lib, kw, status):
    assert mgrouped_dgd(lib, **kw) == status
    assert "te_fp8_mgrouped_gemm_dgrad_deterministic" in lib.te_last_error_message().decode()


def test_mgrouped_dgrad_deterministic_workspace_is_the_dense_size(lib):
    # one row of N (padded to 4) fp32 column sums per 64 token rows, as the dense call
    assert lib.te_fp8_dgrad_bgrad_workspace_bytes(512, 256) == 8 * 256 * 4
    assert lib.te_fp8_dgrad_bgrad_workspace_bytes(512, 250) == 8 * 252 * 4


@pytest.mark.parametrize("kw,status", [
    (dict(mb=0), INV), (dict(mb=MB + 2), MISAL), (dict(G=0), INV), (dict(G=1025), INV), (dict(sum_m=0), INV),
    (dict(sum_m=300), INV), (dict(K=100), INV), (dict(epi=8), INV), (dict(epi=4), INV), (dict(epi=1), INV),
    (dict(bias=BIAS), INV), (dict(epi=1, bias=BIAS, N=250, ldy=252), MISAL), (dict(epi=1, bias=BIAS + 8), MISAL),
    (dict(y=0), INV), (dict(ydt=1), INV), (dict(ldy=128), INV), (dict(pre=Z, ldpre=256), INV),
    (dict(epi=6, pre=0), INV), (dict(accum=0), INV),
])
def test_mgrouped_rejects(lib, kw, status):
    assert mgrouped(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(gk=0), INV), (dict(G=0), INV), (dict(G=257), INV), (dict(sum_k=0), INV), (dict(sum_k=200), INV),
    (dict(M=0), INV), (dict(out=0), INV), (dict(accum=0), INV), (dict(gk=GK + 4), MISAL),
])
def test_kgrouped_device_sizes_rejects(lib, kw, status):
    assert kgrouped_dev(lib, **kw) == status


def cast(lib, x=A, rows=4, cols=256, ldx=256, dt=1, flags=0, q=B, ldq=256, s=S):
    return lib.te_cast_fp8_per_token(p(x), rows, cols, ldx, dt, flags, p(q), ldq, p(s), None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=0), INV), (dict(q=0), INV), (dict(s=0), INV), (dict(rows=0), INV),
    (dict(cols=100), INV), (dict(cols=0), INV), (dict(ldx=128), INV), (dict(ldq=128), INV),
    (dict(dt=3), INV), (dict(flags=2), INV),
    (dict(x=MIS), MISAL), (dict(ldx=260), MISAL), (dict(q=MIS), MISAL), (dict(ldq=264), MISAL), (dict(s=S + 1), MISAL),
    (dict(s=S + 4), MISAL),
])
def test_cast_rejects(lib, kw, status):
    assert cast(lib, **kw) == status


class CastOp(ctypes.Structure):
    _fields_ = [("x_bf16", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld_x", ctypes.c_int64), ("q", ctypes.c_void_p), ("ld_q", ctypes.c_int64),
                ("scales", ctypes.c_void_p)]


def cast_batch(lib, ops, n=None, dt=1, flags=0):
    arr = (CastOp * max(1, len(ops)))(*[CastOp(*o) for o in ops])
    return lib.te_cast_fp8_per_token_batch(ctypes.cast(arr, ctypes.c_void_p), len(ops) if n is None else n, dt, flags,
                                           None)


GOOD = (A, 4, 256, 256, B, 256, S)


@pytest.mark.parametrize("ops,n,dt,flags,status", [
    ([GOOD], 0, 1, 0, INV), ([GOOD] * 9, None, 1, 0, INV), ([GOOD], None, 3, 0, INV), ([GOOD], None, 1, 2, INV),
    ([GOOD, (A, 4, 100, 256, B, 256, S)], None, 1, 0, INV), ([GOOD, (0, 4, 256, 256, B, 256, S)], None, 1, 0, INV),
    ([(A, 0, 256, 256, B, 256, S)], None, 1, 0, INV), ([GOOD, (MIS, 4, 256, 256, B, 256, S)], None, 1, 0, MISAL),
    ([(A, 4, 256, 256, B, 264, S)], None, 1, 0, MISAL), ([(A, 4, 256, 256, B, 256, S + 4)], None, 1, 0, MISAL),
])
def test_cast_batch_rejects(lib, ops, n, dt, flags, status):
    assert cast_batch(lib, ops, n, dt, flags) == status


def test_cast_batch_null_ops(lib):
    assert lib.te_cast_fp8_per_token_batch(None, 1, 1, 0, None) == INV


QT = 0x70000
ST = 0x80000


def cast_t(lib, x=A, rows=256, cols=384, ldx=384, dt=1, flags=0, q=B, ldq=384, s=S, qt=QT, ldqt=256, st=ST):
    return lib.te_cast_fp8_per_token_transpose(p(x), rows, cols, ldx, dt, flags, p(q), ldq, p(s), p(qt), ldqt,
                                               p(st), None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=0), INV), (dict(qt=0), INV), (dict(st=0), INV), (dict(q=0), INV), (dict(s=0), INV),
    (dict(rows=0), INV), (dict(rows=100), INV), (dict(rows=200), INV), (dict(cols=100), INV), (dict(cols=0), INV),
    (dict(cols=264, ldx=264, ldq=272), INV), (dict(q=0, s=0, cols=100, ldx=104), INV), (dict(q=0, s=0, cols=0), INV),
    (dict(ldx=256), INV), (dict(ldq=256), INV), (dict(ldqt=128), INV), (dict(dt=3), INV), (dict(flags=2), INV),
    (dict(x=MIS), MISAL), (dict(ldx=388), MISAL), (dict(q=MIS), MISAL), (dict(ldq=392), MISAL),
    (dict(qt=MIS), MISAL), (dict(ldqt=264), MISAL), (dict(s=S + 4), MISAL), (dict(st=ST + 4), MISAL),
])
def test_cast_transpose_rejects(lib, kw, status):
    assert cast_t(lib, **kw) == status


def test_cast_transpose_rowwise_is_optional_but_both_or_neither(lib):
    # q and its scales are given together or not at all (ldq is then ignored)
    assert cast_t(lib, q=0, s=0, ldq=0, x=MIS) == MISAL   # validation reaches the alignment checks
    assert cast_t(lib, q=0, ldq=0) == INV
    assert cast_t(lib, s=0) == INV


@pytest.mark.parametrize("rows,ld", [(0, 0), (1, 4), (3, 4), (4, 4), (5, 8), (7168, 7168), (2113, 2116)])
def test_scale_ld(lib, rows, ld):
    assert lib.te_scale_ld(rows) == ld
    assert te.scale_ld(rows) == ld


def test_binding_checks_scale_shape(lib):
    q = torch.zeros((8, 256), dtype=torch.uint8)
    with pytest.raises(te.TeFp8Error, match="x_scales"):
        te.te_fp8_gemm_fwd(q, torch.zeros((8, 2)), 1, q, torch.zeros((2, 8)), 1)
    with pytest.raises(te.TeFp8Error, match="b_scales"):
        te.te_fp8_wgrad_accum(q, torch.zeros((2, 8)), 1, q, torch.zeros((2, 4)), 1, torch.zeros((8, 8)))


def test_status_strings(lib):
    names = [lib.te_status_string(i).decode() for i in range(6)]
    assert names == ["TE_OK", "TE_ERR_INVALID_ARGUMENT", "TE_ERR_MISALIGNED", "TE_ERR_UNSUPPORTED",
                     "TE_ERR_HIP", "TE_ERR_INTERNAL"]


def test_python_binding_raises_with_message(lib):
    with pytest.raises(te.TeFp8Error) as ei:
        te._check(wgrad(lib, K=100))
    assert "multiple of 128" in str(ei.value) and ei.value.status == INV
