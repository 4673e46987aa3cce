/*
 * te_fp8.h - C ABI of the MI355X (gfx950) scaled-FP8 Linear-layer GEMM library.
 *
 * Five operations make up the FP8 hot path of a transformer Linear layer in
 * training: the per-token fp8 cast that produces the operands, the forward
 * GEMM with its bias/GELU epilogue, the data-gradient GEMM with its dGELU and
 * bias-gradient epilogue, the weight-gradient GEMM that accumulates into an
 * fp32 buffer, and its K-grouped (mixture-of-experts) variant:
 *   te_cast_fp8_per_token, te_fp8_gemm_fwd, te_fp8_gemm_dgrad,
 *   te_fp8_wgrad_accum, te_fp8_kgrouped_wgrad.
 * Around them:
 *   te_cast_fp8_per_token_batch       several casts in one launch
 *   te_cast_fp8_per_token_transpose   the cast and the cast of the transpose
 *                                     (the weight gradient's operand) from one read
 *   te_fp8_gemm_fwd_quant,            the forward / data-gradient result stored
 *   te_fp8_gemm_dgrad_quant           as the next GEMM's fp8 operand
 *   te_fp8_gemm_dgrad_deterministic   the bias gradient without atomics
 *   te_fp8_gemm_dgrad_deterministic_noalloc   the same without a caller workspace
 *                                     (te_fp8_dgrad_bgrad_workspace_bytes)
 *   te_fp8_wgrad_accum_bgrad          the bias gradient beside the weight gradient
 *   te_fp8_kgrouped_wgrad_device_sizes  expert sizes in device memory
 *   te_fp8_mgrouped_gemm_fwd          the experts' forward (and plain data gradient)
 *   te_fp8_mgrouped_gemm_dgrad        the experts' data gradient with dGELU and
 *                                     per-expert bias gradients
 *   te_fp8_mgrouped_gemm_dgrad_deterministic   the same with the per-expert
 *                                     bias gradients summed without atomics
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Layout.   Every matrix is row-major.  Every GEMM is "NT": both operands are
 *            stored contraction-contiguous, A as [M][K] and B as [N][K] with
 *            row stride exactly K bytes, and the result is D[M][N] = A * B^T.
 *            The Linear layer's three products map onto this form as
 *              forward:  A = X   [tokens][in],   B = W   [out][in]
 *              dgrad:    A = dY  [tokens][out],  B = W^T [in][out]
 *              wgrad:    A = dY^T[out][tokens],  B = X^T [in][tokens]
 *            so no GEMM_m/GEMM_n swap between BLAS orders ever arises and the
 *            bias vector always has length N, the output-feature count.
 *  Scales.   Operands are fp8 with one fp32 dequantisation scale per row and
 *            per 128 consecutive contraction elements ("1x128" groups): the
 *            value of element (r, k) is dec(q[r][k]) * s(r, k/128).  The
 *            pages fix one fp32 scale per row and 128-element block but not
 *            where it sits in memory; this library's own choice (not a
 *            statement of the pages) stores them contraction-block-major,
 *            so that a tile's row scales of one block are a single 16-byte
 *            aligned run: s(r, kb) = scales[kb * te_scale_ld(rows) + r], i.e. an
 *            array [K/128][te_scale_ld(rows)] whose row kb holds the scales of
 *            all rows for block kb (entries r >= rows are padding, never
 *            used).  K must be a multiple of 128 and at most 2^22 (for the
 *            K-grouped call: the sum of the groups' K).
 *  Formats.  TE_DTYPE_E4M3 is OCP E4M3FN (max 448), TE_DTYPE_E5M2 is OCP
 *            E5M2 (max 57344).  Any pairing of the two is accepted.
 *  Accumulation policy.  Every GEMM takes an explicit te_accum_t; it is
 *            never inferred from the operand formats.  Both policies compute
 *            the same mathematical result in fp32:
 *              TE_ACCUM_FULL_FP32: each 128-deep block is reduced by the
 *                matrix cores from zero and promoted into the fp32
 *                accumulator with its scale product in vector fp32 FMA.
 *              TE_ACCUM_FAST: an output tile whose row and column scales
 *                over its contraction range are all powers of two (the
 *                TE_CAST_POW2_SCALE cast produces only such scales) has the
 *                scales applied inside the matrix-core instruction and
 *                accumulates in one chain with no vector work; any other tile
 *                falls back to the FULL update, so the result is correct for
 *                any input.
 *  Ownership. Every pointer is device memory owned by the caller, except
 *            group_k, which is host memory read during the call.  The
 *            library allocates nothing, never synchronises, and enqueues its
 *            kernels on `stream` (NULL = the default stream); results are
 *            ready when that stream reaches them.  Outputs must not alias
 *            inputs.
 *  Errors.   Arguments are validated on the host before anything is
 *            enqueued; on any error nothing is launched, no output is
 *            touched, and the call returns a status other than TE_OK.
 *            te_last_error_message() then describes the failure (thread-
 *            local).  A failed launch returns TE_ERR_HIP.  Device faults
 *            surface at the caller's next synchronisation.  No C++ exception
 *            crosses this interface.  Calls are thread-safe; calls that
 *            overlap on one stream are ordered by it.
 *  Alignment. fp8, bf16 and scale base pointers must be 16-byte aligned,
 *            other fp32 pointers 4-byte aligned.
 *  Logging.  With the environment variable TE_FP8_LOG=1 every call prints one
 *            line to stderr (operation, sizes, formats, policy, epilogue,
 *            tile, grid).  Logging never changes results.
 *  Kernels.  A product whose 256 x 256 output tiles number at most a
 *            quarter of the device's compute units runs on a kernel that
 *            gives each 64 x 128 part of a tile a workgroup of its own (the
 *            others: one persistent workgroup per compute unit).  Both
 *            produce the same bits wherever TE_ACCUM_FAST's power-of-two test
 *            agrees (it is taken per output tile of the kernel that runs).
 *            The environment variable TE_FP8_GEMM_PATH=wave or =persistent
 *            forces one of the two for the products the first supports
 *            (every call but the quantising store of the transpose); it is
 *            read on every call.  The tile count of a grouped call is that of
 *            all its groups together.
 *
 * Sources: the Linear layer's forward and backward equations and the bias
 * length are those of the maintainer's explanation on "Replaced cublasLt calls
 * with rocblas gemm + 6 manually crafted epilogues" (ROCm/TransformerEngine
 * pull request 3); the accumulate-into-out weight gradient and its K-grouped
 * form are those of "Weight gradient kernels for dense and MoE models"
 * (DeepGEMM pull request 95); the explicit per-op accumulation precision is
 * that agreed on "FP8 GEMM for the fprop should use fast accumulation"
 * (openxla/xla issue 6168).
 */
#ifndef TE_FP8_H
#define TE_FP8_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TE_OK = 0,
    TE_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, bad enum or flag */
    TE_ERR_MISALIGNED = 2,       /* pointer or stride alignment violated */
    TE_ERR_UNSUPPORTED = 3,      /* a combination this library does not implement */
    TE_ERR_HIP = 4,              /* the HIP runtime reported an error at launch */
    TE_ERR_INTERNAL = 5          /* anything else; a bug */
} te_status_t;

typedef enum {
    TE_DTYPE_E4M3 = 1, /* OCP E4M3FN */
    TE_DTYPE_E5M2 = 2, /* OCP E5M2 */
    TE_DTYPE_BF16 = 3,
    TE_DTYPE_F32 = 4
} te_dtype_t;

/* 0 is deliberately not a policy: a zero-initialised argument is rejected. */
typedef enum {
    TE_ACCUM_FULL_FP32 = 1,
    TE_ACCUM_FAST = 2
} te_accum_t;

/* Epilogue flags.  Forward: BIAS, GELU, AUX_PREACT.  Dgrad: DGELU, BGRAD. */
enum {
    TE_EPI_NONE = 0,
    TE_EPI_BIAS = 1,       /* z = acc + bias[n] (bias bf16, length N) */
    TE_EPI_GELU = 2,       /* y = GELU(z), tanh form */
    TE_EPI_AUX_PREACT = 4, /* also store bf16(z) to preact (needs GELU) */
    TE_EPI_DGELU = 8,      /* D = acc * GELU'(preact[m][n]) */
    TE_EPI_BGRAD = 16      /* bias_grad[n] = sum over m of D (after DGELU) */
};

/* Cast flags. */
enum {
    TE_CAST_POW2_SCALE = 1 /* round every scale up to a power of two */
};

/*
 * Leading dimension, in floats, of the scale array of an operand with `rows`
 * rows: rows rounded up to a multiple of 4, so every block's scales start on
 * a 16-byte boundary.  Returns 0 for rows <= 0.
 */
int64_t te_scale_ld(int64_t rows);

/*
 * Per-token 1x128 cast of a bf16 matrix to fp8 with fp32 scales.
 *
 * The pages name this step (the wgrad example casts both operands with a
 * per-token cast before the GEMM) but do not define it; this is the reading:
 * for every row r and every group g of 128 consecutive columns,
 *     amax   = max |x[r][128g .. 128g+127]|,   amax_c = max(amax, 2^-100)
 *     s      = fl32(amax_c / FP8_MAX)                      (dequant scale)
 *     q[r][k]= enc(fl32(x[r][k] * fl32(FP8_MAX / amax_c)))
 * with fp32 IEEE division and product, and enc() rounding to nearest even and
 * saturating to +-FP8_MAX (sign kept on zero).  With TE_CAST_POW2_SCALE,
 * s = 2^j for the smallest integer j with FP8_MAX * 2^j >= amax_c, and
 * q = enc(x * 2^-j).  Inputs must be finite (otherwise the output is
 * unspecified).
 *
 *  x_bf16   [rows][ld_x] bf16, the first `cols` columns are cast
 *  rows     >= 1;  cols >= 128 and a multiple of 128;  ld_x >= cols, ld_x % 8 == 0
 *  out_dtype TE_DTYPE_E4M3 or TE_DTYPE_E5M2
 *  flags    0 or TE_CAST_POW2_SCALE
 *  q        [rows][ld_q] bytes, ld_q >= cols, ld_q % 16 == 0
 *  scales   [cols/128][te_scale_ld(rows)] fp32 (block-major, see Scales);
 *           padding entries are left untouched
 */
te_status_t te_cast_fp8_per_token(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                  te_dtype_t out_dtype, uint32_t flags, void* q, int64_t ld_q,
                                  float* scales, hipStream_t stream);

/* One operand of te_cast_fp8_per_token_batch (fields as te_cast_fp8_per_token's). */
typedef struct {
    const void* x_bf16;
    int64_t rows, cols, ld_x;
    void* q;
    int64_t ld_q;
    float* scales;
} te_cast_operand_t;

/*
 * Several per-token casts with one format and flags in one launch, e.g. the
 * two operands of a weight gradient: each operand's result is exactly that
 * of te_cast_fp8_per_token on it.  One launch lets a small operand's loads
 * overlap a large one's instead of paying its own start-up and latency.
 *
 *  ops    HOST array of n operands (read during the call), each valid for
 *         te_cast_fp8_per_token; outputs must not overlap
 *  n      1 .. 8
 */
te_status_t te_cast_fp8_per_token_batch(const te_cast_operand_t* ops, int32_t n, te_dtype_t out_dtype,
                                        uint32_t flags, hipStream_t stream);

/*
 * Fused per-token cast and cast-transpose: one read of a bf16 matrix X
 * [rows][cols] produces the operand cast of X (as te_cast_fp8_per_token) and
 * the operand cast of X^T, i.e. 1x128 groups running down the columns of X.
 *
 * Where it sits: for a Linear layer with X [tokens][in] and dY
 * [tokens][out], the weight gradient contracts over tokens (A = dY^T,
 * B = X^T in the NT form above), while the forward and data-gradient GEMMs
 * contract over features (X and dY themselves).  The DeepGEMM weight-gradient
 * page counts the separate per-token casts feeding its kernel among the costs
 * that lower end-to-end performance; this call reads the activation or
 * gradient once and writes both operands.
 *
 * Definition (bit-identical to two separate casts):
 *     (q,  scales)   = te_cast_fp8_per_token(X)        if q != NULL
 *     (qt, scales_t) = te_cast_fp8_per_token(X^T)
 * with the same out_dtype and flags for both.
 *
 *  x_bf16    [rows][ld_x] bf16; rows >= 128 and a multiple of 128; cols a
 *            positive multiple of 128 when q is given, else of 8 (the
 *            transposed groups need only the rows to be whole groups);
 *            ld_x >= cols, ld_x % 8 == 0
 *  q         [rows][ld_q] bytes, ld_q >= cols, ld_q % 16 == 0, or NULL
 *  scales    [cols/128][te_scale_ld(rows)] fp32; NULL iff q is NULL
 *  qt        [cols][ld_qt] bytes, ld_qt >= rows, ld_qt % 16 == 0
 *  scales_t  [rows/128][te_scale_ld(cols)] fp32
 *  Errors as for te_cast_fp8_per_token.
 */
te_status_t te_cast_fp8_per_token_transpose(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                            te_dtype_t out_dtype, uint32_t flags, void* q, int64_t ld_q,
                                            float* scales, void* qt, int64_t ld_qt, float* scales_t,
                                            hipStream_t stream);

/*
 * Forward GEMM of a Linear layer, Y = X * W^T + b, with fused epilogues.
 *   acc[m][n] = sum_k x[m][k] w[n][k]      (dequantised, fp32 accumulation)
 *   z = acc + bias[n]          if TE_EPI_BIAS, else acc
 *   y = GELU(z)                if TE_EPI_GELU, else z
 *   preact[m][n] = bf16(z)     if TE_EPI_AUX_PREACT (requires TE_EPI_GELU)
 *
 *  x, x_scales   [M][K] fp8, [K/128][te_scale_ld(M)] fp32
 *  w, w_scales   [N][K] fp8, [K/128][te_scale_ld(N)] fp32
 *  bias_bf16     [N] bf16, required iff TE_EPI_BIAS
 *  y             [M][ld_y], y_dtype TE_DTYPE_BF16 or TE_DTYPE_F32, ld_y >= N
 *                (ld_y % 8 == 0 for bf16, % 4 == 0 for fp32)
 *  preact_bf16   [M][ld_preact] bf16, required iff TE_EPI_AUX_PREACT
 *  M, N >= 1; K >= 128, K % 128 == 0
 */
te_status_t te_fp8_gemm_fwd(const void* x, const float* x_scales, te_dtype_t x_dtype,
                            const void* w, const float* w_scales, te_dtype_t w_dtype,
                            int64_t M, int64_t N, int64_t K,
                            const void* bias_bf16, uint32_t epilogue,
                            void* y, te_dtype_t y_dtype, int64_t ld_y,
                            void* preact_bf16, int64_t ld_preact,
                            te_accum_t accum, hipStream_t stream);

/*
 * The forward GEMM with a quantising store: the fp32 result of the forward
 * epilogue (the y of te_fp8_gemm_fwd before any rounding) is written as the
 * per-token cast the next FP8 Linear layer consumes, with no bf16 round trip
 * and no separate cast (the DeepGEMM weight-gradient page counts the unfused
 * casts around its kernel among the end-to-end costs):
 *   (q, q_scales)   = te_cast_fp8_per_token applied to y[M][N] in fp32
 *   (qt, qt_scales) = te_cast_fp8_per_token applied to y^T[N][M] in fp32
 * i.e. 1x128 groups along N (the next layer's forward operand) and/or along
 * M (the tokens: the operand that layer's weight gradient contracts over,
 * what te_cast_fp8_per_token_transpose makes from a bf16 y), the same scale
 * and rounding rules, with q_dtype and cast_flags (0 or TE_CAST_POW2_SCALE)
 * as the cast takes them.  preact (TE_EPI_AUX_PREACT) is stored as in
 * te_fp8_gemm_fwd.  Either output pair may be null, not both.
 *
 *  x, w, bias, epilogue, preact, accum   as te_fp8_gemm_fwd;  N % 128 == 0
 *  q         [M][ld_q] bytes, ld_q >= N, ld_q % 16 == 0
 *  q_scales  [N/128][te_scale_ld(M)] fp32 (block-major); padding untouched
 *  qt        [N][ld_qt] bytes, ld_qt >= M, ld_qt % 16 == 0; needs M % 128 == 0
 *  qt_scales [M/128][te_scale_ld(N)] fp32 (block-major); padding untouched
 */
te_status_t te_fp8_gemm_fwd_quant(const void* x, const float* x_scales, te_dtype_t x_dtype,
                                  const void* w, const float* w_scales, te_dtype_t w_dtype,
                                  int64_t M, int64_t N, int64_t K,
                                  const void* bias_bf16, uint32_t epilogue,
                                  te_dtype_t q_dtype, uint32_t cast_flags, void* q, int64_t ld_q, float* q_scales,
                                  void* qt, int64_t ld_qt, float* qt_scales,
                                  void* preact_bf16, int64_t ld_preact,
                                  te_accum_t accum, hipStream_t stream);

/*
 * Data-gradient GEMM of a Linear layer with its backward epilogues
 * (dX = dY * W, and for the layer before a GELU, the gradient through it):
 *   acc[m][n] = sum_k dy[m][k] wt[n][k]
 *   D = acc * GELU'(preact[m][n])   if TE_EPI_DGELU, else acc
 *   bias_grad[n] = sum_m D[m][n]    if TE_EPI_BGRAD (fp32, before dx rounding;
 *                                   overwritten, not accumulated)
 *   dx[m][n] = D
 * dGELU is applied before the bias gradient.  The bias-gradient sum is formed
 * with atomic fp32 additions, so its last bits may vary from run to run.
 *
 *  dy, dy_scales [M][K] fp8 (typically E5M2), [K/128][te_scale_ld(M)]
 *  wt, wt_scales [N][K] fp8 (W^T re-cast along the out dimension), [K/128][te_scale_ld(N)]
 *  preact_bf16   [M][ld_preact] bf16, required iff TE_EPI_DGELU
 *  bias_grad     [N] fp32, required iff TE_EPI_BGRAD
 *  dx            [M][ld_dx], dx_dtype TE_DTYPE_BF16 or TE_DTYPE_F32
 */
te_status_t te_fp8_gemm_dgrad(const void* dy, const float* dy_scales, te_dtype_t dy_dtype,
                              const void* wt, const float* wt_scales, te_dtype_t wt_dtype,
                              int64_t M, int64_t N, int64_t K, uint32_t epilogue,
                              const void* preact_bf16, int64_t ld_preact,
                              float* bias_grad,
                              void* dx, te_dtype_t dx_dtype, int64_t ld_dx,
                              te_accum_t accum, hipStream_t stream);

/*
 * Bytes of workspace te_fp8_gemm_dgrad_deterministic needs for an M x N
 * output: one row of N fp32 column sums (padded to a multiple of 4) per 64
 * output rows, i.e. ceil(M/256) * 4 * roundup(N, 4) * 4.  0 for M or N < 1.
 */
int64_t te_fp8_dgrad_bgrad_workspace_bytes(int64_t M, int64_t N);

/*
 * te_fp8_gemm_dgrad with a run-to-run deterministic bias gradient: instead of
 * fp32 atomics, every 64-row slice of D stores its column sums to a row of the
 * caller's workspace, and a second kernel sums those rows in a fixed order
 * (bias_grad is overwritten).  The epilogue must include TE_EPI_BGRAD.  The
 * pages place the bias gradient's reduction in the library (BGRADB among the
 * cuBLASLt-style epilogues); this is its atomic-free form.
 *
 *  workspace        device memory, 16-byte aligned, at least
 *                   te_fp8_dgrad_bgrad_workspace_bytes(M, N) bytes
 *                   (contents on entry irrelevant; clobbered)
 *  everything else  as te_fp8_gemm_dgrad
 */
te_status_t te_fp8_gemm_dgrad_deterministic(const void* dy, const float* dy_scales, te_dtype_t dy_dtype,
                                            const void* wt, const float* wt_scales, te_dtype_t wt_dtype,
                                            int64_t M, int64_t N, int64_t K, uint32_t epilogue,
                                            const void* preact_bf16, int64_t ld_preact,
                                            float* bias_grad, void* workspace, int64_t workspace_bytes,
                                            void* dx, te_dtype_t dx_dtype, int64_t ld_dx,
                                            te_accum_t accum, hipStream_t stream);

/*
 * te_fp8_gemm_dgrad_deterministic for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and the same result, bit for bit, with
 * the column-sum workspace taken from a static array inside the library
 * instead of from the caller.  The call allocates nothing.
 *
 *  Limit      te_fp8_dgrad_bgrad_workspace_bytes(M, N) must not exceed
 *             TE_NOALLOC_SCRATCH_BYTES (8 MiB, e.g. M = 8192 with N up to
 *             16384); larger outputs are rejected (TE_ERR_INVALID_ARGUMENT)
 *             before anything is enqueued.
 *  Sharing    each GPU holds one such array for the life of the process and
 *             every call on that GPU uses it: calls that can overlap on one GPU
 *             (different streams, no ordering between them) race and give
 *             undefined bias gradients; calls ordered on one stream are safe.
 *             Nothing in the array has to start at zero (every slot the
 *             reduction reads is written by the same call first).
 *  Arguments  as te_fp8_gemm_dgrad_deterministic without the workspace.
 */
#define TE_NOALLOC_SCRATCH_BYTES (8 << 20)
te_status_t te_fp8_gemm_dgrad_deterministic_noalloc(const void* dy, const float* dy_scales, te_dtype_t dy_dtype,
                                                    const void* wt, const float* wt_scales, te_dtype_t wt_dtype,
                                                    int64_t M, int64_t N, int64_t K, uint32_t epilogue,
                                                    const void* preact_bf16, int64_t ld_preact, float* bias_grad,
                                                    void* dx, te_dtype_t dx_dtype, int64_t ld_dx,
                                                    te_accum_t accum, hipStream_t stream);

/*
 * The data-gradient GEMM with a quantising store: D (after dGELU) is written
 * as its per-token cast along N, e.g. the e5m2 dZ the next data-gradient
 * GEMM consumes, instead of dx; the bias gradient is formed from the fp32 D
 * as in te_fp8_gemm_dgrad.
 *   (q, q_scales)   = te_cast_fp8_per_token applied to D[M][N] in fp32
 *   (qt, qt_scales) = te_cast_fp8_per_token applied to D^T[N][M] in fp32
 * (e.g. e5m2 dZ for the data gradient of the layer before, and dZ^T along
 * the tokens for its weight gradient).
 *
 *  dy, wt, epilogue, preact, bias_grad, accum   as te_fp8_gemm_dgrad;  N % 128 == 0
 *  q_dtype, cast_flags, q, ld_q, q_scales,
 *  qt, ld_qt, qt_scales                          as te_fp8_gemm_fwd_quant
 */
te_status_t te_fp8_gemm_dgrad_quant(const void* dy, const float* dy_scales, te_dtype_t dy_dtype,
                                    const void* wt, const float* wt_scales, te_dtype_t wt_dtype,
                                    int64_t M, int64_t N, int64_t K, uint32_t epilogue,
                                    const void* preact_bf16, int64_t ld_preact, float* bias_grad,
                                    te_dtype_t q_dtype, uint32_t cast_flags, void* q, int64_t ld_q, float* q_scales,
                                    void* qt, int64_t ld_qt, float* qt_scales,
                                    te_accum_t accum, hipStream_t stream);

/*
 * Weight-gradient GEMM that accumulates: out[m][n] += sum_k a[m][k] b[n][k].
 * The product is formed in fp32 from zero and added to out once (one fp32
 * rounding of the sum), as the gradient of a weight accumulates over
 * micro-batches.  A second identical call adds the product again.
 *
 *  a, a_scales   [M][K] fp8 (dY^T, cast along tokens), [K/128][te_scale_ld(M)]
 *  b, b_scales   [N][K] fp8 (X^T, cast along tokens), [K/128][te_scale_ld(N)]
 *  out           [M][ld_out] fp32, ld_out >= N, read and written
 */
te_status_t te_fp8_wgrad_accum(const void* a, const float* a_scales, te_dtype_t a_dtype,
                               const void* b, const float* b_scales, te_dtype_t b_dtype,
                               int64_t M, int64_t N, int64_t K,
                               float* out, int64_t ld_out,
                               te_accum_t accum, hipStream_t stream);

/*
 * The weight gradient with the bias gradient taken from its own operand: the
 * reduction over tokens that gives the bias gradient is the row sum of
 * A = dY^T, so the call adds
 *   bias_grad[m] = sum_k a[m][k]     (dequantised fp8 A, fp32; overwritten)
 * to te_fp8_wgrad_accum's out += A * B^T.  The pages place the bias
 * gradient's reduction in the GEMM library next to the weight-gradient GEMM
 * (the BGRADB epilogue among the cuBLASLt-style ones); here it is a second,
 * HBM-bound kernel over A's codes and scales (K + K/32 bytes per row).  It
 * sums the fp8 operand, so it differs from the sum of the bf16 gradient by
 * the cast's rounding (half an fp8 ulp per element at most).
 *
 *  bias_grad  [M] fp32, 4-byte aligned
 *  everything else as te_fp8_wgrad_accum
 */
te_status_t te_fp8_wgrad_accum_bgrad(const void* a, const float* a_scales, te_dtype_t a_dtype,
                                     const void* b, const float* b_scales, te_dtype_t b_dtype,
                                     int64_t M, int64_t N, int64_t K,
                                     float* out, int64_t ld_out, float* bias_grad,
                                     te_accum_t accum, hipStream_t stream);

/*
 * K-grouped weight gradient for mixture-of-experts layers: expert g owns the
 * contraction columns [off_g, off_g + K_g) of both operands, off_g being the
 * sum of the earlier K's, and
 *   out[g][m][n] += sum_{k in group g} a[m][k] b[n][k].
 * A group with K_g = 0 leaves out[g] untouched.
 *
 *  a, a_scales   [M][sumK] fp8, [sumK/128][te_scale_ld(M)]
 *  b, b_scales   [N][sumK] fp8, [sumK/128][te_scale_ld(N)]
 *  group_k       HOST array of G int64, each >= 0 and a multiple of 128,
 *                sumK = their sum >= 128
 *  G             1 .. 1024
 *  out           [G][M][N] fp32, contiguous
 */
te_status_t te_fp8_kgrouped_wgrad(const void* a, const float* a_scales, te_dtype_t a_dtype,
                                  const void* b, const float* b_scales, te_dtype_t b_dtype,
                                  int64_t M, int64_t N, const int64_t* group_k, int32_t G,
                                  float* out, te_accum_t accum, hipStream_t stream);

/*
 * The same K-grouped weight gradient with the group sizes in device memory,
 * e.g. the per-expert token counts a router produced on the GPU: nothing is
 * read back to the host and the call does not synchronise.  The pages name
 * the grouped weight-gradient kernel but not where its group sizes live;
 * reading them on the device is this library's own design choice.
 *
 *  a, a_scales   [M][sum_k] fp8, [sum_k/128][te_scale_ld(M)]
 *  b, b_scales   [N][sum_k] fp8, [sum_k/128][te_scale_ld(N)]
 *  sum_k         the operands' contraction width: >= 128, a multiple of 128
 *  group_k_device DEVICE array of G int64 (8-byte aligned), read by the
 *                kernel when it runs: each >= 0 and a multiple of 128, summing
 *                to at most sum_k (columns past the sum are not used).  Other
 *                values give unspecified results, but every offset and length
 *                is clamped to the operands, so no read leaves them.
 *  G             1 .. 256
 *  out           [G][M][N] fp32, contiguous; a group with K_g = 0 is left
 *                untouched
 * Tiles are scheduled in group order (the host-sized call orders groups
 * longest first, which balances unequal groups better).
 */
te_status_t te_fp8_kgrouped_wgrad_device_sizes(const void* a, const float* a_scales, te_dtype_t a_dtype,
                                               const void* b, const float* b_scales, te_dtype_t b_dtype,
                                               int64_t M, int64_t N, int64_t sum_k, const int64_t* group_k_device,
                                               int32_t G, float* out, te_accum_t accum, hipStream_t stream);

/*
 * M-grouped forward GEMM for mixture-of-experts layers (also the data
 * gradient, with each expert's W^T as w and no epilogue): the tokens are
 * sorted by expert into blocks of 256 rows (each expert's rows padded to a
 * multiple of 256), and block i uses expert e = m_block_group[i]:
 *   y[m][n] = epi( sum_k x[m][k] w[e][n][k] (+ bias[e][n]) ),  m in block i
 * with the epilogues of te_fp8_gemm_fwd.  A block whose entry is outside
 * [0, G) (e.g. -1 for padding) is skipped: its rows of y (and preact) are not
 * written.  The expert of each block is read from device memory when the
 * kernel runs (no host synchronisation).  The pages' grouped GEMMs are the
 * K-grouped weight gradient; this is its forward/data-gradient counterpart
 * over the same per-expert token layout.
 *
 *  x, x_scales     [sum_m][K] fp8, [K/128][te_scale_ld(sum_m)]
 *  w, w_scales     [G][N][K] fp8, [G][K/128][te_scale_ld(N)] (each expert's
 *                  operand and scales as te_fp8_gemm_fwd takes them)
 *  sum_m           >= 256, a multiple of 256;  N >= 1;  K as te_fp8_gemm_fwd
 *  G               1 .. 1024
 *  m_block_group   DEVICE array of sum_m/256 int32 (4-byte aligned)
 *  bias_bf16       [G][N] bf16, required iff TE_EPI_BIAS (then N % 8 == 0)
 *  y, preact_bf16  as te_fp8_gemm_fwd, [sum_m][ld]
 */
te_status_t te_fp8_mgrouped_gemm_fwd(const void* x, const float* x_scales, te_dtype_t x_dtype,
                                     const void* w, const float* w_scales, te_dtype_t w_dtype,
                                     int64_t sum_m, int64_t N, int64_t K, int32_t G, const int32_t* m_block_group,
                                     const void* bias_bf16, uint32_t epilogue,
                                     void* y, te_dtype_t y_dtype, int64_t ld_y,
                                     void* preact_bf16, int64_t ld_preact,
                                     te_accum_t accum, hipStream_t stream);

/*
 * M-grouped data gradient with the backward epilogues of te_fp8_gemm_dgrad,
 * per expert: block i of 256 token rows uses expert e = m_block_group[i]'s
 * W^T, and
 *   D = dy * wt[e]^T, D *= GELU'(preact) (TE_EPI_DGELU, preact [sum_m][ld]),
 *   bias_grad[e][n] = sum of D[m][n] over the rows m of expert e's blocks
 *                     (TE_EPI_BGRAD; fp32 atomics; all G rows overwritten,
 *                     an expert with no block gets zeros),
 *   dx = D.  Blocks outside [0, G) are skipped (their dx rows not written).
 *
 *  dy, dy_scales   [sum_m][K] fp8, [K/128][te_scale_ld(sum_m)]
 *  wt, wt_scales   [G][N][K] fp8, [G][K/128][te_scale_ld(N)]
 *  bias_grad       [G][N] fp32, required iff TE_EPI_BGRAD
 *  everything else as te_fp8_mgrouped_gemm_fwd / te_fp8_gemm_dgrad
 */
te_status_t te_fp8_mgrouped_gemm_dgrad(const void* dy, const float* dy_scales, te_dtype_t dy_dtype,
                                       const void* wt, const float* wt_scales, te_dtype_t wt_dtype,
                                       int64_t sum_m, int64_t N, int64_t K, int32_t G, const int32_t* m_block_group,
                                       uint32_t epilogue, const void* preact_bf16, int64_t ld_preact,
                                       float* bias_grad, void* dx, te_dtype_t dx_dtype, int64_t ld_dx,
                                       te_accum_t accum, hipStream_t stream);

/*
 * te_fp8_mgrouped_gemm_dgrad with run-to-run deterministic per-expert bias
 * gradients, as te_fp8_gemm_dgrad_deterministic does it for the dense call:
 * every 64-row slice of D stores its column sums to a row of the caller's
 * workspace, and a second kernel sums, for each expert e and column n, the
 * rows of expert e's blocks in block order (bias_grad is overwritten; an
 * expert with no block gets zeros; a skipped block's rows are neither written
 * nor read).  The epilogue must include TE_EPI_BGRAD.
 *
 *  workspace        device memory, 16-byte aligned, at least
 *                   te_fp8_dgrad_bgrad_workspace_bytes(sum_m, N) bytes
 *                   (contents on entry irrelevant; clobbered)
 *  everything else  as te_fp8_mgrouped_gemm_dgrad
 */
te_status_t te_fp8_mgrouped_gemm_dgrad_deterministic(const void* dy, const float* dy_scales, te_dtype_t dy_dtype,
                                                     const void* wt, const float* wt_scales, te_dtype_t wt_dtype,
                                                     int64_t sum_m, int64_t N, int64_t K, int32_t G,
                                                     const int32_t* m_block_group, uint32_t epilogue,
                                                     const void* preact_bf16, int64_t ld_preact, float* bias_grad,
                                                     void* workspace, int64_t workspace_bytes, void* dx,
                                                     te_dtype_t dx_dtype, int64_t ld_dx, te_accum_t accum,
                                                     hipStream_t stream);

/* Static description of a status code. */
const char* te_status_string(te_status_t status);

/* Detail of the calling thread's most recent failure ("" if none). */
const char* te_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* TE_FP8_H */
