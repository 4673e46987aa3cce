"""Python binding of the gfx950 scaled-FP8 Linear-layer GEMM library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libte_fp8.so`` behind the C ABI declared in ``include/te_fp8.h``.
PyTorch supplies device memory and the current stream.  There is no fallback:
if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libte_fp8.so")

# te_status_t
TE_OK = 0
# te_dtype_t
TE_DTYPE_E4M3 = 1
TE_DTYPE_E5M2 = 2
TE_DTYPE_BF16 = 3
TE_DTYPE_F32 = 4
# te_accum_t
TE_ACCUM_FULL_FP32 = 1
TE_ACCUM_FAST = 2
# epilogue flags
TE_EPI_NONE = 0
TE_EPI_BIAS = 1
TE_EPI_GELU = 2
TE_EPI_AUX_PREACT = 4
TE_EPI_DGELU = 8
TE_EPI_BGRAD = 16
# cast flags
TE_CAST_POW2_SCALE = 1

EXPORTED = ("te_cast_fp8_per_token", "te_cast_fp8_per_token_batch", "te_cast_fp8_per_token_transpose", "te_fp8_gemm_fwd", "te_fp8_gemm_fwd_quant",
            "te_fp8_gemm_dgrad_quant", "te_fp8_gemm_dgrad_deterministic", "te_fp8_dgrad_bgrad_workspace_bytes",
            "te_fp8_gemm_dgrad_deterministic_noalloc",
            "te_fp8_wgrad_accum_bgrad", "te_fp8_gemm_dgrad", "te_fp8_wgrad_accum",
            "te_fp8_kgrouped_wgrad", "te_fp8_kgrouped_wgrad_device_sizes", "te_fp8_mgrouped_gemm_fwd",
            "te_fp8_mgrouped_gemm_dgrad",
            "te_fp8_mgrouped_gemm_dgrad_deterministic",
            "te_status_string", "te_last_error_message", "te_scale_ld")


class TeFp8Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def load_library():
    """Load libte_fp8.so (built in-tree by ``fp8_linear_layer_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m fp8_linear_layer_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, U32, I32, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_int32, ctypes.c_int
    lib.te_status_string.restype = ctypes.c_char_p
    lib.te_status_string.argtypes = [I]
    lib.te_last_error_message.restype = ctypes.c_char_p
    lib.te_last_error_message.argtypes = []
    lib.te_scale_ld.restype = I64
    lib.te_scale_ld.argtypes = [I64]
    lib.te_cast_fp8_per_token.restype = I
    lib.te_cast_fp8_per_token.argtypes = [P, I64, I64, I64, I, U32, P, I64, P, P]
    lib.te_cast_fp8_per_token_batch.restype = I
    lib.te_cast_fp8_per_token_batch.argtypes = [P, I32, I, U32, P]
    lib.te_cast_fp8_per_token_transpose.restype = I
    lib.te_cast_fp8_per_token_transpose.argtypes = [P, I64, I64, I64, I, U32, P, I64, P, P, I64, P, P]
    lib.te_fp8_gemm_fwd.restype = I
    lib.te_fp8_gemm_fwd.argtypes = [P, P, I, P, P, I, I64, I64, I64, P, U32, P, I, I64, P, I64, I, P]
    lib.te_fp8_gemm_fwd_quant.restype = I
    lib.te_fp8_gemm_fwd_quant.argtypes = [P, P, I, P, P, I, I64, I64, I64, P, U32, I, U32, P, I64, P, P, I64, P, P,
                                          I64, I, P]
    lib.te_fp8_gemm_dgrad_quant.restype = I
    lib.te_fp8_gemm_dgrad_quant.argtypes = [P, P, I, P, P, I, I64, I64, I64, U32, P, I64, P, I, U32, P, I64, P, P,
                                            I64, P, I, P]
    lib.te_fp8_dgrad_bgrad_workspace_bytes.restype = I64
    lib.te_fp8_dgrad_bgrad_workspace_bytes.argtypes = [I64, I64]
    lib.te_fp8_gemm_dgrad_deterministic.restype = I
    lib.te_fp8_gemm_dgrad_deterministic.argtypes = [P, P, I, P, P, I, I64, I64, I64, U32, P, I64, P, P, I64, P, I,
                                                    I64, I, P]
    lib.te_fp8_gemm_dgrad_deterministic_noalloc.restype = I
    lib.te_fp8_gemm_dgrad_deterministic_noalloc.argtypes = [P, P, I, P, P, I, I64, I64, I64, U32, P, I64, P, P, I,
                                                            I64, I, P]
    lib.te_fp8_gemm_dgrad.restype = I
    lib.te_fp8_gemm_dgrad.argtypes = [P, P, I, P, P, I, I64, I64, I64, U32, P, I64, P, P, I, I64, I, P]
    lib.te_fp8_wgrad_accum.restype = I
    lib.te_fp8_wgrad_accum.argtypes = [P, P, I, P, P, I, I64, I64, I64, P, I64, I, P]
    lib.te_fp8_wgrad_accum_bgrad.restype = I
    lib.te_fp8_wgrad_accum_bgrad.argtypes = [P, P, I, P, P, I, I64, I64, I64, P, I64, P, I, P]
    lib.te_fp8_kgrouped_wgrad.restype = I
    lib.te_fp8_kgrouped_wgrad.argtypes = [P, P, I, P, P, I, I64, I64, P, I32, P, I, P]
    lib.te_fp8_kgrouped_wgrad_device_sizes.restype = I
    lib.te_fp8_kgrouped_wgrad_device_sizes.argtypes = [P, P, I, P, P, I, I64, I64, I64, P, I32, P, I, P]
    lib.te_fp8_mgrouped_gemm_fwd.restype = I
    lib.te_fp8_mgrouped_gemm_fwd.argtypes = [P, P, I, P, P, I, I64, I64, I64, I32, P, P, U32, P, I, I64, P, I64, I, P]
    lib.te_fp8_mgrouped_gemm_dgrad.restype = I
    lib.te_fp8_mgrouped_gemm_dgrad.argtypes = [P, P, I, P, P, I, I64, I64, I64, I32, P, U32, P, I64, P, P, I, I64, I,
                                               P]
    lib.te_fp8_mgrouped_gemm_dgrad_deterministic.restype = I
    lib.te_fp8_mgrouped_gemm_dgrad_deterministic.argtypes = [P, P, I, P, P, I, I64, I64, I64, I32, P, U32, P, I64, P,
                                                             P, I64, P, I, I64, I, P]
    _lib = lib
    return lib


def _check(status: int):
    if status != TE_OK:
        lib = load_library()
        msg = lib.te_last_error_message().decode()
        raise TeFp8Error(status, f"{lib.te_status_string(status).decode()}: {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _cols(t):
    return t.shape[-1]


# --------------------------------------------------------------- entry points
def scale_ld(rows: int) -> int:
    """Leading dimension of the block-major scales of an operand with `rows` rows (te_scale_ld)."""
    return int(load_library().te_scale_ld(int(rows)))


def _scales_ok(t, rows, k, name):
    """The kernels read scales of K/128 blocks at stride scale_ld(rows); refuse anything smaller."""
    want = (k // 128, scale_ld(rows))
    if t is None or t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != want:
        raise TeFp8Error(1, f"{name}: expected contiguous fp32 scales of shape {want} "
                         f"(got {None if t is None else (tuple(t.shape), t.dtype)})")


def te_cast_fp8_per_token(x, out_dtype=TE_DTYPE_E4M3, flags=0, q=None, scales=None, stream=None):
    """bf16 x [rows, cols] -> (q uint8 [rows, cols], scales fp32 [cols/128, scale_ld(rows)], block-major:
    the scale of row r and 128-column block kb is scales[kb, r])."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((cols // 128, scale_ld(rows)), dtype=torch.float32, device=x.device)
    _scales_ok(scales, rows, cols, "scales")
    _check(load_library().te_cast_fp8_per_token(_ptr(x), rows, cols, x.stride(0), out_dtype, flags,
                                                _ptr(q), q.stride(0), _ptr(scales), _stream(stream)))
    return q, scales


class _CastOperand(ctypes.Structure):
    _fields_ = [("x_bf16", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld_x", ctypes.c_int64), ("q", ctypes.c_void_p), ("ld_q", ctypes.c_int64),
                ("scales", ctypes.c_void_p)]


_CAST_ARRAYS = {}  # one reusable operand array per batch size (calls on one thread at a time)


def te_cast_fp8_per_token_batch(xs, out_dtype=TE_DTYPE_E4M3, flags=0, qs=None, scales=None, stream=None):
    """The per-token cast of every bf16 matrix in xs in one launch; returns [(q, scales), ...]."""
    n = len(xs)
    arr = _CAST_ARRAYS.get(n)
    if arr is None:
        arr = _CAST_ARRAYS[n] = (_CastOperand * n)()
    out = []
    for i, x in enumerate(xs):
        assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
        rows, cols = x.shape
        q = qs[i] if qs is not None and qs[i] is not None else \
            torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
        sc = scales[i] if scales is not None and scales[i] is not None else \
            torch.empty((cols // 128, scale_ld(rows)), dtype=torch.float32, device=x.device)
        _scales_ok(sc, rows, cols, "scales")
        o = arr[i]
        o.x_bf16, o.rows, o.cols, o.ld_x = x.data_ptr(), rows, cols, x.stride(0)
        o.q, o.ld_q, o.scales = q.data_ptr(), q.stride(0), sc.data_ptr()
        out.append((q, sc))
    _check(load_library().te_cast_fp8_per_token_batch(arr, n, out_dtype, flags, _stream(stream)))
    return out


def te_cast_fp8_per_token_transpose(x, out_dtype=TE_DTYPE_E4M3, flags=0, rowwise=True, q=None, scales=None,
                                    qt=None, scales_t=None, stream=None):
    """bf16 x [rows, cols] -> (q, scales, qt, scales_t): the per-token cast of x (None, None when
    rowwise is False) and of x^T, from one read of x.  qt is uint8 [cols, rows]; scales_t is
    block-major fp32 [rows/128, scale_ld(cols)]."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    rows, cols = x.shape
    if rowwise:
        if q is None:
            q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
        if scales is None:
            scales = torch.empty((cols // 128, scale_ld(rows)), dtype=torch.float32, device=x.device)
        _scales_ok(scales, rows, cols, "scales")
    else:
        q = scales = None
    if qt is None:
        qt = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    if scales_t is None:
        scales_t = torch.empty((rows // 128, scale_ld(cols)), dtype=torch.float32, device=x.device)
    _scales_ok(scales_t, cols, rows, "scales_t")
    _check(load_library().te_cast_fp8_per_token_transpose(
        _ptr(x), rows, cols, x.stride(0), out_dtype, flags, _ptr(q), q.stride(0) if q is not None else 0,
        _ptr(scales), _ptr(qt), qt.stride(0), _ptr(scales_t), _stream(stream)))
    return q, scales, qt, scales_t


def te_fp8_gemm_fwd(x, x_scales, x_dtype, w, w_scales, w_dtype, bias=None, epilogue=TE_EPI_NONE,
                    y=None, y_dtype=TE_DTYPE_BF16, preact=None, accum=TE_ACCUM_FAST, stream=None):
    """Y[M,N] = epi(X[M,K] W[N,K]^T (+ b)); returns y (and fills preact if given)."""
    M, K = x.shape
    N = w.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16 if y_dtype == TE_DTYPE_BF16 else torch.float32, device=x.device)
    _scales_ok(x_scales, M, K, "x_scales")
    _scales_ok(w_scales, N, K, "w_scales")
    _check(load_library().te_fp8_gemm_fwd(
        _ptr(x), _ptr(x_scales), x_dtype, _ptr(w), _ptr(w_scales), w_dtype, M, N, K,
        _ptr(bias), epilogue, _ptr(y), y_dtype, y.stride(0),
        _ptr(preact), preact.stride(0) if preact is not None else 0, accum, _stream(stream)))
    return y


def _quant_outputs(M, N, device, rowwise, transposed, q, q_scales, qt, qt_scales):
    if rowwise:
        if q is None:
            q = torch.empty((M, N), dtype=torch.uint8, device=device)
        if q_scales is None:
            q_scales = torch.empty((N // 128, scale_ld(M)), dtype=torch.float32, device=device)
        _scales_ok(q_scales, M, N, "q_scales")
    else:
        q = q_scales = None
    if transposed:
        if qt is None:
            qt = torch.empty((N, M), dtype=torch.uint8, device=device)
        if qt_scales is None:
            qt_scales = torch.empty((M // 128, scale_ld(N)), dtype=torch.float32, device=device)
        _scales_ok(qt_scales, N, M, "qt_scales")
    else:
        qt = qt_scales = None
    return q, q_scales, qt, qt_scales


def te_fp8_gemm_fwd_quant(x, x_scales, x_dtype, w, w_scales, w_dtype, bias=None, epilogue=TE_EPI_NONE,
                          q_dtype=TE_DTYPE_E4M3, cast_flags=0, q=None, q_scales=None, preact=None,
                          accum=TE_ACCUM_FAST, stream=None, rowwise=True, transposed=False, qt=None,
                          qt_scales=None):
    """The forward GEMM whose fp32 result is stored as its per-token cast (rowwise: 1x128 groups
    along N) and/or the cast of its transpose (transposed: groups along M, qt [N, M]).  Returns
    (q, q_scales), or (q, q_scales, qt, qt_scales) when transposed."""
    M, K = x.shape
    N = w.shape[0]
    _scales_ok(x_scales, M, K, "x_scales")
    _scales_ok(w_scales, N, K, "w_scales")
    q, q_scales, qt, qt_scales = _quant_outputs(M, N, x.device, rowwise, transposed, q, q_scales, qt, qt_scales)
    _check(load_library().te_fp8_gemm_fwd_quant(
        _ptr(x), _ptr(x_scales), x_dtype, _ptr(w), _ptr(w_scales), w_dtype, M, N, K,
        _ptr(bias), epilogue, q_dtype, cast_flags, _ptr(q), q.stride(0) if q is not None else 0, _ptr(q_scales),
        _ptr(qt), qt.stride(0) if qt is not None else 0, _ptr(qt_scales),
        _ptr(preact), preact.stride(0) if preact is not None else 0, accum, _stream(stream)))
    return (q, q_scales, qt, qt_scales) if transposed else (q, q_scales)


def te_fp8_gemm_dgrad(dy, dy_scales, dy_dtype, wt, wt_scales, wt_dtype, epilogue=TE_EPI_NONE, preact=None,
                      bias_grad=None, dx=None, dx_dtype=TE_DTYPE_BF16, accum=TE_ACCUM_FULL_FP32, stream=None):
    """D[M,N] = dY[M,K] Wt[N,K]^T, then dGELU / bias-grad; returns dx."""
    M, K = dy.shape
    N = wt.shape[0]
    if dx is None:
        dx = torch.empty((M, N), dtype=torch.bfloat16 if dx_dtype == TE_DTYPE_BF16 else torch.float32, device=dy.device)
    _scales_ok(dy_scales, M, K, "dy_scales")
    _scales_ok(wt_scales, N, K, "wt_scales")
    _check(load_library().te_fp8_gemm_dgrad(
        _ptr(dy), _ptr(dy_scales), dy_dtype, _ptr(wt), _ptr(wt_scales), wt_dtype, M, N, K, epilogue,
        _ptr(preact), preact.stride(0) if preact is not None else 0, _ptr(bias_grad),
        _ptr(dx), dx_dtype, dx.stride(0), accum, _stream(stream)))
    return dx


def te_fp8_wgrad_accum(a, a_scales, a_dtype, b, b_scales, b_dtype, out, accum=TE_ACCUM_FULL_FP32, stream=None):
    """out[M,N] += A[M,K] B[N,K]^T in fp32; returns out."""
    M, K = a.shape
    N = b.shape[0]
    _scales_ok(a_scales, M, K, "a_scales")
    _scales_ok(b_scales, N, K, "b_scales")
    _check(load_library().te_fp8_wgrad_accum(
        _ptr(a), _ptr(a_scales), a_dtype, _ptr(b), _ptr(b_scales), b_dtype, M, N, K,
        _ptr(out), out.stride(0), accum, _stream(stream)))
    return out


def te_fp8_kgrouped_wgrad(a, a_scales, a_dtype, b, b_scales, b_dtype, group_k, out,
                          accum=TE_ACCUM_FULL_FP32, stream=None):
    """out[g] += A[:, group g] B[:, group g]^T; group_k is a host sequence of ints."""
    M = a.shape[0]
    N = b.shape[0]
    gk = (ctypes.c_int64 * len(group_k))(*[int(k) for k in group_k])
    _scales_ok(a_scales, M, sum(gk), "a_scales")
    _scales_ok(b_scales, N, sum(gk), "b_scales")
    _check(load_library().te_fp8_kgrouped_wgrad(
        _ptr(a), _ptr(a_scales), a_dtype, _ptr(b), _ptr(b_scales), b_dtype, M, N,
        ctypes.cast(gk, ctypes.c_void_p), len(group_k), _ptr(out), accum, _stream(stream)))
    return out


def te_fp8_kgrouped_wgrad_device_sizes(a, a_scales, a_dtype, b, b_scales, b_dtype, group_k, out,
                                       accum=TE_ACCUM_FULL_FP32, stream=None):
    """out[g] += A[:, off_g:off_g+K_g] B[:, off_g:off_g+K_g]^T with group_k an int64 tensor on the device
    (read by the kernel; nothing is copied to the host)."""
    M, S = a.shape
    N = b.shape[0]
    assert group_k.dtype == torch.int64 and group_k.is_cuda and group_k.dim() == 1 and group_k.is_contiguous()
    G = group_k.numel()
    assert out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (G, M, N)
    _scales_ok(a_scales, M, S, "a_scales")
    _scales_ok(b_scales, N, S, "b_scales")
    _check(load_library().te_fp8_kgrouped_wgrad_device_sizes(
        _ptr(a), _ptr(a_scales), a_dtype, _ptr(b), _ptr(b_scales), b_dtype, M, N, S, _ptr(group_k), G,
        _ptr(out), accum, _stream(stream)))
    return out


def te_fp8_mgrouped_gemm_fwd(x, x_scales, x_dtype, w, w_scales, w_dtype, m_block_group, bias=None,
                             epilogue=TE_EPI_NONE, y=None, y_dtype=TE_DTYPE_BF16, preact=None, accum=TE_ACCUM_FAST,
                             stream=None):
    """y[m] = epi(x[m] w[e]^T (+ bias[e])) for the rows m of every 256-row block whose expert
    e = m_block_group[block] is in [0, G); w is [G, N, K] fp8 with scales [G, K/128, scale_ld(N)]."""
    sum_m, K = x.shape
    G, N, K2 = w.shape
    assert K2 == K and w.is_contiguous()
    assert m_block_group.dtype == torch.int32 and m_block_group.is_cuda and m_block_group.is_contiguous()
    assert m_block_group.numel() * 256 == sum_m
    want = (G, K // 128, scale_ld(N))
    if w_scales.dtype != torch.float32 or not w_scales.is_contiguous() or tuple(w_scales.shape) != want:
        raise TeFp8Error(1, f"w_scales: expected contiguous fp32 scales of shape {want}")
    _scales_ok(x_scales, sum_m, K, "x_scales")
    if y is None:
        y = torch.empty((sum_m, N), dtype=torch.bfloat16 if y_dtype == TE_DTYPE_BF16 else torch.float32,
                        device=x.device)
    _check(load_library().te_fp8_mgrouped_gemm_fwd(
        _ptr(x), _ptr(x_scales), x_dtype, _ptr(w), _ptr(w_scales), w_dtype, sum_m, N, K, G, _ptr(m_block_group),
        _ptr(bias), epilogue, _ptr(y), y_dtype, y.stride(0),
        _ptr(preact), preact.stride(0) if preact is not None else 0, accum, _stream(stream)))
    return y


def te_fp8_gemm_dgrad_quant(dy, dy_scales, dy_dtype, wt, wt_scales, wt_dtype, epilogue=TE_EPI_NONE, preact=None,
                            bias_grad=None, q_dtype=TE_DTYPE_E5M2, cast_flags=0, q=None, q_scales=None,
                            accum=TE_ACCUM_FULL_FP32, stream=None, rowwise=True, transposed=False, qt=None,
                            qt_scales=None):
    """The data-gradient GEMM whose fp32 D (after dGELU) is stored as its per-token cast and/or the
    cast of its transpose (as te_fp8_gemm_fwd_quant); bias_grad is filled as by te_fp8_gemm_dgrad."""
    M, K = dy.shape
    N = wt.shape[0]
    _scales_ok(dy_scales, M, K, "dy_scales")
    _scales_ok(wt_scales, N, K, "wt_scales")
    q, q_scales, qt, qt_scales = _quant_outputs(M, N, dy.device, rowwise, transposed, q, q_scales, qt, qt_scales)
    _check(load_library().te_fp8_gemm_dgrad_quant(
        _ptr(dy), _ptr(dy_scales), dy_dtype, _ptr(wt), _ptr(wt_scales), wt_dtype, M, N, K, epilogue,
        _ptr(preact), preact.stride(0) if preact is not None else 0, _ptr(bias_grad), q_dtype, cast_flags,
        _ptr(q), q.stride(0) if q is not None else 0, _ptr(q_scales),
        _ptr(qt), qt.stride(0) if qt is not None else 0, _ptr(qt_scales), accum, _stream(stream)))
    return (q, q_scales, qt, qt_scales) if transposed else (q, q_scales)


def te_fp8_gemm_dgrad_deterministic(dy, dy_scales, dy_dtype, wt, wt_scales, wt_dtype, bias_grad,
                                    epilogue=TE_EPI_BGRAD, preact=None, workspace=None, dx=None,
                                    dx_dtype=TE_DTYPE_BF16, accum=TE_ACCUM_FULL_FP32, stream=None):
    """te_fp8_gemm_dgrad with the bias gradient summed in a fixed order through a workspace
    (allocated here when not given); returns dx."""
    M, K = dy.shape
    N = wt.shape[0]
    _scales_ok(dy_scales, M, K, "dy_scales")
    _scales_ok(wt_scales, N, K, "wt_scales")
    lib = load_library()
    need = int(lib.te_fp8_dgrad_bgrad_workspace_bytes(M, N))
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dy.device)
    if dx is None:
        dx = torch.empty((M, N), dtype=torch.bfloat16 if dx_dtype == TE_DTYPE_BF16 else torch.float32, device=dy.device)
    _check(lib.te_fp8_gemm_dgrad_deterministic(
        _ptr(dy), _ptr(dy_scales), dy_dtype, _ptr(wt), _ptr(wt_scales), wt_dtype, M, N, K, epilogue,
        _ptr(preact), preact.stride(0) if preact is not None else 0, _ptr(bias_grad), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(dx), dx_dtype, dx.stride(0), accum, _stream(stream)))
    return dx


NOALLOC_SCRATCH_BYTES = 8 << 20  # TE_NOALLOC_SCRATCH_BYTES


def te_fp8_gemm_dgrad_deterministic_noalloc(dy, dy_scales, dy_dtype, wt, wt_scales, wt_dtype, bias_grad, dx,
                                            epilogue=TE_EPI_BGRAD, preact=None, dx_dtype=TE_DTYPE_BF16,
                                            accum=TE_ACCUM_FULL_FP32, stream=None):
    """te_fp8_gemm_dgrad_deterministic with the column-sum workspace in the library's static scratch
    (the call allocates nothing; dx and bias_grad are the caller's); returns dx."""
    M, K = dy.shape
    N = wt.shape[0]
    _scales_ok(dy_scales, M, K, "dy_scales")
    _scales_ok(wt_scales, N, K, "wt_scales")
    _check(load_library().te_fp8_gemm_dgrad_deterministic_noalloc(
        _ptr(dy), _ptr(dy_scales), dy_dtype, _ptr(wt), _ptr(wt_scales), wt_dtype, M, N, K, epilogue,
        _ptr(preact), preact.stride(0) if preact is not None else 0, _ptr(bias_grad), _ptr(dx), dx_dtype,
        dx.stride(0), accum, _stream(stream)))
    return dx


def te_fp8_mgrouped_gemm_dgrad(dy, dy_scales, dy_dtype, wt, wt_scales, wt_dtype, m_block_group,
                               epilogue=TE_EPI_NONE, preact=None, bias_grad=None, dx=None, dx_dtype=TE_DTYPE_BF16,
                               accum=TE_ACCUM_FULL_FP32, stream=None):
    """dx[m] = (dy[m] wt[e]^T) * GELU'(preact[m]) for each 256-row block's expert e, with per-expert
    bias gradients bias_grad[e] = column sums over expert e's rows; returns dx."""
    sum_m, K = dy.shape
    G, N, K2 = wt.shape
    assert K2 == K and wt.is_contiguous()
    assert m_block_group.dtype == torch.int32 and m_block_group.is_cuda and m_block_group.is_contiguous()
    assert m_block_group.numel() * 256 == sum_m
    want = (G, K // 128, scale_ld(N))
    if wt_scales.dtype != torch.float32 or not wt_scales.is_contiguous() or tuple(wt_scales.shape) != want:
        raise TeFp8Error(1, f"wt_scales: expected contiguous fp32 scales of shape {want}")
    _scales_ok(dy_scales, sum_m, K, "dy_scales")
    if bias_grad is not None:
        assert bias_grad.dtype == torch.float32 and bias_grad.is_contiguous() and bias_grad.numel() == G * N
    if dx is None:
        dx = torch.empty((sum_m, N), dtype=torch.bfloat16 if dx_dtype == TE_DTYPE_BF16 else torch.float32,
                         device=dy.device)
    _check(load_library().te_fp8_mgrouped_gemm_dgrad(
        _ptr(dy), _ptr(dy_scales), dy_dtype, _ptr(wt), _ptr(wt_scales), wt_dtype, sum_m, N, K, G, _ptr(m_block_group),
        epilogue, _ptr(preact), preact.stride(0) if preact is not None else 0, _ptr(bias_grad), _ptr(dx), dx_dtype,
        dx.stride(0), accum, _stream(stream)))
    return dx


def te_fp8_mgrouped_gemm_dgrad_deterministic(dy, dy_scales, dy_dtype, wt, wt_scales, wt_dtype, m_block_group,
                                             bias_grad, epilogue=TE_EPI_BGRAD, preact=None, workspace=None, dx=None,
                                             dx_dtype=TE_DTYPE_BF16, accum=TE_ACCUM_FULL_FP32, stream=None):
    """te_fp8_mgrouped_gemm_dgrad with the per-expert bias gradients summed in a fixed order through a
    workspace (allocated here when not given); returns dx."""
    sum_m, K = dy.shape
    G, N, K2 = wt.shape
    assert K2 == K and wt.is_contiguous()
    assert m_block_group.dtype == torch.int32 and m_block_group.is_cuda and m_block_group.is_contiguous()
    assert m_block_group.numel() * 256 == sum_m
    want = (G, K // 128, scale_ld(N))
    if wt_scales.dtype != torch.float32 or not wt_scales.is_contiguous() or tuple(wt_scales.shape) != want:
        raise TeFp8Error(1, f"wt_scales: expected contiguous fp32 scales of shape {want}")
    _scales_ok(dy_scales, sum_m, K, "dy_scales")
    assert bias_grad.dtype == torch.float32 and bias_grad.is_contiguous() and bias_grad.numel() == G * N
    lib = load_library()
    need = int(lib.te_fp8_dgrad_bgrad_workspace_bytes(sum_m, N))
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dy.device)
    if dx is None:
        dx = torch.empty((sum_m, N), dtype=torch.bfloat16 if dx_dtype == TE_DTYPE_BF16 else torch.float32,
                         device=dy.device)
    _check(lib.te_fp8_mgrouped_gemm_dgrad_deterministic(
        _ptr(dy), _ptr(dy_scales), dy_dtype, _ptr(wt), _ptr(wt_scales), wt_dtype, sum_m, N, K, G, _ptr(m_block_group),
        epilogue, _ptr(preact), preact.stride(0) if preact is not None else 0, _ptr(bias_grad), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(dx), dx_dtype, dx.stride(0), accum, _stream(stream)))
    return dx


def te_fp8_wgrad_accum_bgrad(a, a_scales, a_dtype, b, b_scales, b_dtype, out, bias_grad,
                             accum=TE_ACCUM_FULL_FP32, stream=None):
    """out += A B^T and bias_grad[m] = sum_k A[m, k] (dequantised); returns out."""
    M, K = a.shape
    N = b.shape[0]
    _scales_ok(a_scales, M, K, "a_scales")
    _scales_ok(b_scales, N, K, "b_scales")
    assert bias_grad.dtype == torch.float32 and bias_grad.numel() >= M
    _check(load_library().te_fp8_wgrad_accum_bgrad(
        _ptr(a), _ptr(a_scales), a_dtype, _ptr(b), _ptr(b_scales), b_dtype, M, N, K, _ptr(out), out.stride(0),
        _ptr(bias_grad), accum, _stream(stream)))
    return out
