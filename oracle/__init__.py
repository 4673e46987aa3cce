"""CPU oracle for the scaled-FP8 Linear GEMMs (fp64, plain definitions).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the library itself never does.
The arithmetic lives in ``oracle.c`` (plain C, double precision); this module
only builds/loads it and marshals numpy arrays.  It shares no code with the HIP
path.  See the header of ``oracle.c`` for the passages each function follows
and for the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

E4M3 = 1
E5M2 = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so (IEEE arithmetic: no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    lib.oracle_fp8_decode.restype = ctypes.c_double
    lib.oracle_fp8_decode.argtypes = [ctypes.c_uint8, I]
    lib.oracle_fp8_encode.restype = ctypes.c_uint8
    lib.oracle_fp8_encode.argtypes = [ctypes.c_float, I]
    lib.oracle_fp8_max.restype = ctypes.c_double
    lib.oracle_fp8_max.argtypes = [I]
    lib.oracle_fp8_decode_array.argtypes = [P, I64, I, P]
    lib.oracle_fp8_encode_array.argtypes = [P, I64, I, P]
    lib.oracle_cast_per_token.restype = I
    lib.oracle_cast_per_token.argtypes = [P, I64, I64, I64, I, I, P, I64, P]
    lib.oracle_cast_per_token_f32.restype = I
    lib.oracle_cast_per_token_f32.argtypes = [P, I64, I64, I64, I, I, P, I64, P]
    lib.oracle_gemm_nt.argtypes = [P, P, I, I64, I64, P, P, I, I64, I64, I64, I64, I64, I64, P, P]
    lib.oracle_gemm_nt_entries.argtypes = [P, P, I, I64, I64, P, P, I, I64, I64, I64, I64,
                                           P, P, I64, P, P]
    lib.oracle_gelu.restype = ctypes.c_double
    lib.oracle_gelu.argtypes = [ctypes.c_double]
    lib.oracle_dgelu.restype = ctypes.c_double
    lib.oracle_dgelu.argtypes = [ctypes.c_double]
    lib.oracle_fwd_epilogue.argtypes = [P, P, I64, I64, P, I, P, P, P]
    lib.oracle_dgrad_epilogue.argtypes = [P, P, I64, I64, P, I64, P, P, P, P]
    lib.oracle_wgrad.argtypes = [P, P, P, I64, I64, I64, P, P]
    lib.oracle_kgrouped_wgrad.argtypes = [P, P, I, P, P, I, I64, I64, P, I, P, P, P]
    lib.oracle_num_threads.restype = I
    _lib = lib
    return lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


# ------------------------------------------------------------------ codecs
def fp8_max(fmt: int) -> float:
    return float(_load().oracle_fp8_max(fmt))


def decode(codes, fmt: int) -> np.ndarray:
    """Exact float64 value of each fp8 code (OCP E4M3FN / E5M2)."""
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().oracle_fp8_decode_array(_p(c), c.size, fmt, _p(out))
    return out


def encode(values, fmt: int) -> np.ndarray:
    """fp32 -> fp8 code: round to nearest even, saturate to the largest finite code."""
    v = _c(values, np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().oracle_fp8_encode_array(_p(v), v.size, fmt, _p(out))
    return out


def bf16_to_f32(bits) -> np.ndarray:
    b = _c(bits, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------ cast
def cast_per_token(x_bf16_bits, fmt: int, pow2: bool = False):
    """Per-token 1x128 cast of a bf16 [rows, cols] array (given as uint16 bits).

    Returns (q uint8 [rows, cols], s float32 [rows, cols/128]).
    """
    x = _c(x_bf16_bits, np.uint16)
    rows, cols = x.shape
    if cols % 128:
        raise ValueError("cols must be a multiple of 128")
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // 128), np.float32)
    rc = _load().oracle_cast_per_token(_p(x), rows, cols, cols, fmt, int(bool(pow2)), _p(q), cols, _p(s))
    if rc != 0:
        raise ValueError("non-finite input to the per-token cast")
    return q, s


def cast_per_token_f32(x, fmt: int, pow2: bool = False):
    """The per-token cast of an fp32 [rows, cols] array (the same fp32 operations as
    cast_per_token, on values that need not be bf16).  Returns (q, s), s row-major."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    if cols % 128:
        raise ValueError("cols must be a multiple of 128")
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // 128), np.float32)
    rc = _load().oracle_cast_per_token_f32(_p(x), rows, cols, cols, fmt, int(bool(pow2)), _p(q), cols, _p(s))
    if rc != 0:
        raise ValueError("non-finite input to the per-token cast")
    return q, s


def cast_per_token_transpose(x_bf16_bits, fmt: int, pow2: bool = False):
    """The per-token cast of x and of its transpose, by definition: (q, s) =
    cast(x), (qt, st) = cast(x^T), where x^T's 1x128 groups run down the
    columns of x (the weight gradient contracts over the token rows).
    Returns (q, s, qt, st), scales row-major as in cast_per_token; q and s are
    None when the column count is not a multiple of 128 (no row-wise groups)."""
    x = _c(x_bf16_bits, np.uint16)
    q, s = cast_per_token(x, fmt, pow2) if x.shape[1] % 128 == 0 else (None, None)
    qt, st = cast_per_token(np.ascontiguousarray(x.T), fmt, pow2)
    return q, s, qt, st


def operand_row_sums(q, s, fmt: int):
    """sum_k dec(q[r, k]) * s[r, k/128] per row, in fp64 (the bias gradient as the row sums of the
    fp8 operand dY^T); also the |.|-magnitude of each sum.  Scales row-major [rows][K/128]."""
    q = _c(q, np.uint8)
    s = _c(s, np.float32).astype(np.float64)
    rows, K = q.shape
    dec = decode(q, fmt).reshape(rows, K // 128, 128)
    return (dec.sum(-1) * s).sum(-1), (np.abs(dec).sum(-1) * s).sum(-1)


# ------------------------------------------------------------------ GEMM
def gemm_nt(qa, sa, fa, qb, sb, fb, k0: int = 0, K: int | None = None):
    """o[m,n] = sum_kb sA sB sum_k dec(qa[m,k]) dec(qb[n,k]); d = same with |terms|."""
    qa = _c(qa, np.uint8); qb = _c(qb, np.uint8)
    sa = _c(sa, np.float32); sb = _c(sb, np.float32)
    M, KA = qa.shape
    N, KB = qb.shape
    assert KA == KB and KA % 128 == 0
    if K is None:
        K = KA - k0
    o = np.empty((M, N), np.float64)
    d = np.empty((M, N), np.float64)
    _load().oracle_gemm_nt(_p(qa), _p(sa), fa, KA, sa.shape[1], _p(qb), _p(sb), fb, KB, sb.shape[1],
                           M, N, k0, K, _p(o), _p(d))
    return o, d


def gemm_nt_entries(qa, sa, fa, qb, sb, fb, mi, ni, k0: int = 0, K: int | None = None):
    """The product of gemm_nt at positions (mi[i], ni[i]) only."""
    qa = _c(qa, np.uint8); qb = _c(qb, np.uint8)
    sa = _c(sa, np.float32); sb = _c(sb, np.float32)
    mi = _c(mi, np.int64); ni = _c(ni, np.int64)
    KA = qa.shape[1]
    if K is None:
        K = KA - k0
    o = np.empty(mi.shape, np.float64)
    d = np.empty(mi.shape, np.float64)
    _load().oracle_gemm_nt_entries(_p(qa), _p(sa), fa, KA, sa.shape[1], _p(qb), _p(sb), fb, qb.shape[1],
                                   sb.shape[1], k0, K, _p(mi), _p(ni), mi.size, _p(o), _p(d))
    return o, d


# ------------------------------------------------------------- epilogues
def gelu(z: float) -> float:
    return float(_load().oracle_gelu(float(z)))


def dgelu(z: float) -> float:
    return float(_load().oracle_dgelu(float(z)))


def fwd_epilogue(o, d, bias_bits=None, gelu_on: bool = False):
    """z = o + b[n]; y = GELU(z) if gelu_on else z.  Returns (y, z, zmag)."""
    o = _c(o, np.float64); d = _c(d, np.float64)
    M, N = o.shape
    b = None if bias_bits is None else _c(bias_bits, np.uint16)
    if b is not None:
        assert b.shape == (N,)
    z = np.empty_like(o); zmag = np.empty_like(o); y = np.empty_like(o)
    _load().oracle_fwd_epilogue(_p(o), _p(d), M, N, _p(b), int(bool(gelu_on)), _p(z), _p(zmag), _p(y))
    return y, z, zmag


def mgrouped_fwd(qx, sx, fx, qw, sw, fw, m_block_group, bias_bits=None, gelu_on: bool = False, block: int = 256):
    """The M-grouped forward by definition: every `block`-row slice of x whose expert e =
    m_block_group[i] is in [0, G) goes through gemm_nt with w[e] and fwd_epilogue with bias[e]
    (expert weights qw [G, N, K], row-major scales sw [G, N, K/128]).  Returns (y, z, zmag) with
    NaN in the rows of skipped blocks."""
    qx = _c(qx, np.uint8); sx = _c(sx, np.float32)
    G, N, _ = qw.shape
    M = qx.shape[0]
    y = np.full((M, N), np.nan); z = np.full((M, N), np.nan); zm = np.full((M, N), np.nan)
    for i, e in enumerate(np.asarray(m_block_group)):
        if not 0 <= e < G:
            continue
        r = slice(i * block, (i + 1) * block)
        o, d = gemm_nt(qx[r], sx[r], fx, qw[e], sw[e], fw)
        y[r], z[r], zm[r] = fwd_epilogue(o, d, None if bias_bits is None else bias_bits[e], gelu_on)
    return y, z, zm


def mgrouped_dgrad(qa, sa, fa, qw, sw, fw, m_block_group, preact_bits=None, block: int = 256):
    """The M-grouped data gradient by definition: every `block`-row slice of the gradient qa whose
    expert e = m_block_group[i] is in [0, G) goes through gemm_nt with the expert's transposed
    weight qw[e] and dgrad_epilogue (GELU' of its pre-activation rows, if given); expert e's bias
    gradient is the sum of its blocks' column sums, zero for an expert with no block.  Returns
    (D, Dmag, db [G, N], dbmag [G, N]) with NaN in the rows of skipped blocks."""
    qa = _c(qa, np.uint8); sa = _c(sa, np.float32)
    G, N, _ = qw.shape
    M = qa.shape[0]
    D = np.full((M, N), np.nan); Dm = np.full((M, N), np.nan)
    db = np.zeros((G, N)); dbm = np.zeros((G, N))
    for i, e in enumerate(np.asarray(m_block_group)):
        if not 0 <= e < G:
            continue
        r = slice(i * block, (i + 1) * block)
        o, d = gemm_nt(qa[r], sa[r], fa, qw[e], sw[e], fw)
        D[r], Dm[r], dbi, dbmi = dgrad_epilogue(o, d, None if preact_bits is None else preact_bits[r], True)
        db[e] += dbi
        dbm[e] += dbmi
    return D, Dm, db, dbm


def dgrad_epilogue(o, d, preact_bits=None, bgrad: bool = False):
    """D = o * GELU'(z) (if preact given); db = column sums of D.  Returns (D, Dmag, db, dbmag)."""
    o = _c(o, np.float64); d = _c(d, np.float64)
    M, N = o.shape
    z = None if preact_bits is None else _c(preact_bits, np.uint16)
    D = np.empty_like(o); Dm = np.empty_like(o)
    db = np.empty(N, np.float64) if bgrad else None
    dbm = np.empty(N, np.float64) if bgrad else None
    _load().oracle_dgrad_epilogue(_p(o), _p(d), M, N, _p(z), N, _p(D), _p(Dm), _p(db), _p(dbm))
    return D, Dm, db, dbm


def wgrad(o, d, out_init):
    """out' = out_init + o; mag = |out_init| + d."""
    o = _c(o, np.float64); d = _c(d, np.float64)
    oi = _c(out_init, np.float32)
    M, N = o.shape
    on = np.empty_like(o); mg = np.empty_like(o)
    _load().oracle_wgrad(_p(o), _p(d), _p(oi), M, N, N, _p(on), _p(mg))
    return on, mg


def kgrouped_wgrad(qa, sa, fa, qb, sb, fb, group_k, out_init):
    """out[g] += A[:, group g] B[:, group g]^T over contiguous column groups."""
    qa = _c(qa, np.uint8); qb = _c(qb, np.uint8)
    sa = _c(sa, np.float32); sb = _c(sb, np.float32)
    gk = _c(group_k, np.int64)
    oi = _c(out_init, np.float32)
    M, N = qa.shape[0], qb.shape[0]
    G = gk.size
    assert oi.shape == (G, M, N) and int(gk.sum()) == qa.shape[1] == qb.shape[1]
    on = np.empty(oi.shape, np.float64); mg = np.empty(oi.shape, np.float64)
    _load().oracle_kgrouped_wgrad(_p(qa), _p(sa), fa, _p(qb), _p(sb), fb, M, N, _p(gk), G,
                                  _p(oi), _p(on), _p(mg))
    return on, mg
