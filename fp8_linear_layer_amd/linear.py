"""Training modules on the C ABI: an FP8 Linear layer and an FP8 MLP block (fc1 -> GELU -> fc2).

Every arithmetic step of the forward and backward passes is a library call (the per-token casts,
the GEMMs and their epilogues); torch supplies device memory, streams and autograd's bookkeeping.
The split follows the functional forward / backward structure of a Linear layer's autograd
function discussed on "How can we use te.Linear with weight parallel?" (TransformerEngine issue
1532), with the backward products of "Replaced cublasLt calls with rocblas gemm + 6 manually
crafted epilogues" (dX = dY W, dW = dY^T X, db = column sums of dY; dGELU before the bias
gradient):

  forward   x -> (x_q, x^T_q)            one cast-transpose of x (e4m3)
            y = x_q W_q^T + b            te_fp8_gemm_fwd: fast accumulation (the fprop policy of
                                         "FP8 GEMM for the fprop should use fast accumulation")
                                         with pow2_scales, where the blocks chain through the
                                         matrix core; FULL on the default IEEE scales, where FAST
                                         would run the same promotion after a scale test
  backward  dy -> (dy_q, dy^T_q)         one cast-transpose of dy (e5m2)
            dW += dy^T_q x^T_q^T, db     te_fp8_wgrad_accum_bgrad (fp32 accumulation into
                                         weight.main_grad, FULL policy), db from the fp8 dy^T
            dx = dy_q (W^T)_q^T          te_fp8_gemm_dgrad, FULL policy

In the MLP block the GELU between the two layers is fused into the library's epilogues: fc1's
forward stores GELU(z) and the pre-activation z, and fc2's data gradient applies GELU'(z) and
forms fc1's bias gradient in its epilogue (DGELU | BGRAD, summed in a fixed order), so no separate
elementwise pass runs.

The weights' fp8 copies (W cast along its input features for the forward, W^T cast along its
output features for the data gradient) come from an Fp8WeightCache: both from one cast-transpose,
made once and reused until the weight changes (torch bumps a tensor's version on every in-place
update, e.g. an optimizer step), so the micro-batches of one step share them (the maintainer's
remark on the same issue that caching the fp8 weight matters for performance).

Shapes: tokens, input and output features must be multiples of 128 (the 1x128 groups run along
both the token and the feature dimensions).  Weights and activations are bf16.
"""
from __future__ import annotations

import math

import torch

from . import (TE_ACCUM_FAST, TE_ACCUM_FULL_FP32, TE_CAST_POW2_SCALE, TE_DTYPE_BF16, TE_DTYPE_E4M3, TE_DTYPE_E5M2, TE_EPI_AUX_PREACT,
               TE_EPI_BGRAD, TE_EPI_BIAS, TE_EPI_DGELU, TE_EPI_GELU, TE_EPI_NONE, te_cast_fp8_per_token_transpose,
               te_fp8_gemm_dgrad, te_fp8_gemm_dgrad_deterministic, te_fp8_gemm_fwd, te_fp8_wgrad_accum,
               te_fp8_wgrad_accum_bgrad)

FWD_DTYPE = TE_DTYPE_E4M3    # activations and weights
BWD_DTYPE = TE_DTYPE_E5M2    # gradients
# Accumulation policy of the forward GEMMs.  Fast accumulation (the matrix core chaining the
# blocks) applies only where a tile's scales are powers of two; the casts here use IEEE scales,
# on which TE_ACCUM_FAST takes the FULL promotion in every tile after testing the tile's scales,
# so FULL gives the same bits without the test (2-4 % of those GEMMs).
FWD_ACCUM = TE_ACCUM_FULL_FP32


def _fwd_policy(pow2: bool):
    """Cast flags of the forward operands (activations and weights) and the forward GEMMs' policy:
    with power-of-two scales the forward chains the blocks through the matrix core (fast
    accumulation); with IEEE scales it is FULL (FWD_ACCUM)."""
    return (TE_CAST_POW2_SCALE, TE_ACCUM_FAST) if pow2 else (0, FWD_ACCUM)


def _check_dims(*dims):
    for d in dims:
        if d % 128:
            raise ValueError(f"FP8 Linear needs every dimension to be a multiple of 128 (got {d})")


class Fp8WeightCache:
    """The fp8 copies of one weight W [out, in]: (q, s) = W cast along `in` (the forward's B
    operand) and (qt, st) = W^T cast along `out` (the data gradient's B operand), refreshed only when
    the weight's storage or version changes."""

    def __init__(self, pow2: bool = False):
        self.pow2 = pow2    # power-of-two scales (the forward operand of a pow2_scales module)
        self._key = None
        self._val = None
        self.casts = 0      # how many times the weight was cast (for tests and logs)

    def get(self, weight: torch.Tensor):
        key = (weight.data_ptr(), weight._version, tuple(weight.shape))
        if key != self._key:
            q, s, qt, st = te_cast_fp8_per_token_transpose(weight.detach(), FWD_DTYPE,
                                                           TE_CAST_POW2_SCALE if self.pow2 else 0)
            self._val, self._key = (q, s, qt, st), key
            self.casts += 1
        return self._val

    def invalidate(self):
        self._key = self._val = None


def _grad_buffer(weight: torch.Tensor):
    """fp32 buffer the weight gradient accumulates into: weight.main_grad when the module keeps one
    (accumulated over micro-batches), else a fresh zero buffer."""
    mg = getattr(weight, "main_grad", None)
    if mg is not None:
        return mg, True
    return torch.zeros(weight.shape, dtype=torch.float32, device=weight.device), False


class _Fp8LinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, bias, cache: Fp8WeightCache, keep: dict | None, pow2: bool):
        M, K = x.shape
        N = weight.shape[0]
        _check_dims(M, K, N)
        flags, accum = _fwd_policy(pow2)
        qx, sx, qxt, sxt = te_cast_fp8_per_token_transpose(x, FWD_DTYPE, flags)
        qw, sw, _, _ = cache.get(weight)
        y = te_fp8_gemm_fwd(qx, sx, FWD_DTYPE, qw, sw, FWD_DTYPE, bias=bias,
                            epilogue=TE_EPI_BIAS if bias is not None else TE_EPI_NONE, y_dtype=TE_DTYPE_BF16,
                            accum=accum)
        ctx.save_for_backward(qxt, sxt, weight)
        ctx.cache, ctx.has_bias, ctx.keep = cache, bias is not None, keep
        if keep is not None:
            keep.update(qx=qx, sx=sx, qxt=qxt, sxt=sxt)
        return y

    @staticmethod
    def backward(ctx, dy):
        qxt, sxt, weight = ctx.saved_tensors
        dy = dy.contiguous()
        qdy, sdy, qdyt, sdyt = te_cast_fp8_per_token_transpose(dy, BWD_DTYPE)
        _, _, qwt, swt = ctx.cache.get(weight)
        dx = te_fp8_gemm_dgrad(qdy, sdy, BWD_DTYPE, qwt, swt, FWD_DTYPE, dx_dtype=TE_DTYPE_BF16,
                               accum=TE_ACCUM_FULL_FP32)
        wbuf, fused = _grad_buffer(weight)
        db = None
        if ctx.has_bias:
            db = torch.empty((weight.shape[0],), dtype=torch.float32, device=dy.device)
            te_fp8_wgrad_accum_bgrad(qdyt, sdyt, BWD_DTYPE, qxt, sxt, FWD_DTYPE, wbuf, db, TE_ACCUM_FULL_FP32)
        else:
            te_fp8_wgrad_accum(qdyt, sdyt, BWD_DTYPE, qxt, sxt, FWD_DTYPE, wbuf, TE_ACCUM_FULL_FP32)
        if ctx.keep is not None:
            ctx.keep.update(qdy=qdy, sdy=sdy, qdyt=qdyt, sdyt=sdyt, db32=db)
        # (autograd wants the parameters' own dtype; with main_grad the fp32 sum stays there)
        dw = None if fused else wbuf.to(weight.dtype)
        return dx, dw, (db.to(torch.bfloat16) if db is not None else None), None, None, None


class _Fp8MlpFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w1, b1, w2, b2, c1: Fp8WeightCache, c2: Fp8WeightCache, keep: dict | None, pow2: bool):
        M, K = x.shape
        H, N = w1.shape[0], w2.shape[0]
        _check_dims(M, K, H, N)
        flags, accum = _fwd_policy(pow2)
        qx, sx, qxt, sxt = te_cast_fp8_per_token_transpose(x, FWD_DTYPE, flags)
        qw1, sw1, _, _ = c1.get(w1)
        z1 = torch.empty((M, H), dtype=torch.bfloat16, device=x.device)
        h = te_fp8_gemm_fwd(qx, sx, FWD_DTYPE, qw1, sw1, FWD_DTYPE, bias=b1,
                            epilogue=TE_EPI_BIAS | TE_EPI_GELU | TE_EPI_AUX_PREACT, preact=z1,
                            y_dtype=TE_DTYPE_BF16, accum=accum)
        qh, sh, qht, sht = te_cast_fp8_per_token_transpose(h, FWD_DTYPE, flags)
        qw2, sw2, _, _ = c2.get(w2)
        y = te_fp8_gemm_fwd(qh, sh, FWD_DTYPE, qw2, sw2, FWD_DTYPE, bias=b2, epilogue=TE_EPI_BIAS,
                            y_dtype=TE_DTYPE_BF16, accum=accum)
        ctx.save_for_backward(qxt, sxt, z1, qht, sht, w1, w2)
        ctx.c1, ctx.c2, ctx.keep = c1, c2, keep
        if keep is not None:
            keep.update(qx=qx, sx=sx, qxt=qxt, sxt=sxt, z1=z1, h=h, qh=qh, sh=sh, qht=qht, sht=sht)
        return y

    @staticmethod
    def backward(ctx, dy):
        qxt, sxt, z1, qht, sht, w1, w2 = ctx.saved_tensors
        dy = dy.contiguous()
        qdy, sdy, qdyt, sdyt = te_cast_fp8_per_token_transpose(dy, BWD_DTYPE)
        # fc2: weight gradient with its bias gradient; data gradient through fc1's GELU with fc1's bias gradient
        w2buf, f2 = _grad_buffer(w2)
        db2 = torch.empty((w2.shape[0],), dtype=torch.float32, device=dy.device)
        te_fp8_wgrad_accum_bgrad(qdyt, sdyt, BWD_DTYPE, qht, sht, FWD_DTYPE, w2buf, db2, TE_ACCUM_FULL_FP32)
        _, _, qw2t, sw2t = ctx.c2.get(w2)
        # (fc1's bias gradient summed in a fixed order: reproducible from run to run, at the atomic
        # form's speed -- the MLP step measured 3339 us atomic, 3345 us ordered)
        db1 = torch.empty((w1.shape[0],), dtype=torch.float32, device=dy.device)
        dz1 = te_fp8_gemm_dgrad_deterministic(qdy, sdy, BWD_DTYPE, qw2t, sw2t, FWD_DTYPE, db1,
                                              epilogue=TE_EPI_DGELU | TE_EPI_BGRAD, preact=z1,
                                              dx_dtype=TE_DTYPE_BF16, accum=TE_ACCUM_FULL_FP32)
        # fc1
        qdz, sdz, qdzt, sdzt = te_cast_fp8_per_token_transpose(dz1, BWD_DTYPE)
        w1buf, f1 = _grad_buffer(w1)
        te_fp8_wgrad_accum(qdzt, sdzt, BWD_DTYPE, qxt, sxt, FWD_DTYPE, w1buf, TE_ACCUM_FULL_FP32)
        _, _, qw1t, sw1t = ctx.c1.get(w1)
        dx = te_fp8_gemm_dgrad(qdz, sdz, BWD_DTYPE, qw1t, sw1t, FWD_DTYPE, dx_dtype=TE_DTYPE_BF16,
                               accum=TE_ACCUM_FULL_FP32)
        if ctx.keep is not None:
            ctx.keep.update(qdy=qdy, sdy=sdy, qdyt=qdyt, sdyt=sdyt, dz1=dz1, db1_32=db1, db2_32=db2, qdz=qdz,
                            sdz=sdz, qdzt=qdzt, sdzt=sdzt)
        return (dx, None if f1 else w1buf.to(w1.dtype), db1.to(torch.bfloat16), None if f2 else w2buf.to(w2.dtype),
                db2.to(torch.bfloat16), None, None, None, None)


def _init_weight(out_f, in_f, device, gen):
    w = torch.empty((out_f, in_f), dtype=torch.float32, device=device)
    bound = 1.0 / math.sqrt(in_f)
    w.uniform_(-bound, bound, generator=gen)
    return w.to(torch.bfloat16)


class Fp8Linear(torch.nn.Module):
    """y = x W^T + b on the FP8 C ABI.  With fuse_wgrad_accumulation the weight gradient is
    accumulated (+=, fp32) into weight.main_grad across backward passes and weight.grad stays None;
    zero main_grad between optimizer steps.  With pow2_scales the forward operands (x and W) are
    cast with power-of-two scales (the smallest power of two not below amax / FP8_MAX: a coarser
    grid) and the forward GEMM accumulates fast, chaining the blocks through the matrix core;
    the gradients keep IEEE scales and the backward GEMMs FULL."""

    def __init__(self, in_features, out_features, bias=True, device="cuda", fuse_wgrad_accumulation=True,
                 generator=None, pow2_scales=False):
        super().__init__()
        _check_dims(in_features, out_features)
        self.pow2_scales = pow2_scales
        self.weight = torch.nn.Parameter(_init_weight(out_features, in_features, device, generator))
        self.bias = torch.nn.Parameter(torch.zeros(out_features, dtype=torch.bfloat16, device=device)) if bias else None
        if fuse_wgrad_accumulation:
            self.weight.main_grad = torch.zeros((out_features, in_features), dtype=torch.float32, device=device)
        self.cache = Fp8WeightCache(pow2_scales)
        self.keep = None      # a dict here receives the fp8 intermediates of the last pass (tests)

    def forward(self, x):
        shp = x.shape
        y = _Fp8LinearFn.apply(x.reshape(-1, shp[-1]), self.weight, self.bias, self.cache, self.keep,
                               self.pow2_scales)
        return y.reshape(*shp[:-1], y.shape[-1])


class Fp8Mlp(torch.nn.Module):
    """fc2(GELU(fc1(x))) with both GEMMs, the GELU and its derivative, and both bias gradients in
    the library's kernels (see the module docstring); pow2_scales as in Fp8Linear (x, h, W1 and W2
    cast with power-of-two scales, both forward GEMMs fast)."""

    def __init__(self, in_features, hidden_features, out_features=None, device="cuda", fuse_wgrad_accumulation=True,
                 generator=None, pow2_scales=False):
        super().__init__()
        out_features = out_features or in_features
        self.pow2_scales = pow2_scales
        _check_dims(in_features, hidden_features, out_features)
        self.w1 = torch.nn.Parameter(_init_weight(hidden_features, in_features, device, generator))
        self.b1 = torch.nn.Parameter(torch.zeros(hidden_features, dtype=torch.bfloat16, device=device))
        self.w2 = torch.nn.Parameter(_init_weight(out_features, hidden_features, device, generator))
        self.b2 = torch.nn.Parameter(torch.zeros(out_features, dtype=torch.bfloat16, device=device))
        if fuse_wgrad_accumulation:
            self.w1.main_grad = torch.zeros(self.w1.shape, dtype=torch.float32, device=device)
            self.w2.main_grad = torch.zeros(self.w2.shape, dtype=torch.float32, device=device)
        self.c1, self.c2 = Fp8WeightCache(pow2_scales), Fp8WeightCache(pow2_scales)
        self.keep = None

    def forward(self, x):
        shp = x.shape
        y = _Fp8MlpFn.apply(x.reshape(-1, shp[-1]), self.w1, self.b1, self.w2, self.b2, self.c1, self.c2, self.keep,
                            self.pow2_scales)
        return y.reshape(*shp[:-1], y.shape[-1])
