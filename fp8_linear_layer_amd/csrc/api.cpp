// C-ABI front end: argument validation, dispatch, per-call logging.
//
// Every check runs on the host before anything is enqueued, so a rejected call
// launches nothing and touches no output.  The library allocates no memory and
// never synchronises; all work goes onto the caller's stream.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "internal.h"
#include "te_fp8.h"

namespace {

thread_local std::string g_last_error;

te_status_t fail(te_status_t st, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

te_status_t ok()
{
    g_last_error.clear();
    return TE_OK;
}

bool log_enabled()
{
    static const bool on = [] {
        const char* v = std::getenv("TE_FP8_LOG");
        return v && v[0] && std::strcmp(v, "0") != 0;
    }();
    return on;
}

const char* dtype_name(te_dtype_t d)
{
    switch (d) {
    case TE_DTYPE_E4M3: return "e4m3";
    case TE_DTYPE_E5M2: return "e5m2";
    case TE_DTYPE_BF16: return "bf16";
    case TE_DTYPE_F32: return "f32";
    }
    return "?";
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool is_fp8(te_dtype_t d) { return d == TE_DTYPE_E4M3 || d == TE_DTYPE_E5M2; }

int to_fmt(te_dtype_t d) { return d == TE_DTYPE_E4M3 ? tefp8::FMT_E4M3 : tefp8::FMT_E5M2; }

constexpr int64_t kMaxDim = (int64_t)1 << 31;
// A 256-row operand tile is addressed through one buffer resource (< 2 GiB range).
constexpr int64_t kMaxK = (int64_t)1 << 22;

// Checks shared by every GEMM entry point.
te_status_t check_operands(const char* fn, const void* a, const float* sa, te_dtype_t da, const void* b,
                           const float* sb, te_dtype_t db, int64_t M, int64_t N, int64_t K, te_accum_t accum)
{
    if (!a || !sa || !b || !sb) return fail(TE_ERR_INVALID_ARGUMENT, "%s: operand or scale pointer is null", fn);
    if (!is_fp8(da) || !is_fp8(db))
        return fail(TE_ERR_INVALID_ARGUMENT, "%s: operand dtypes must be TE_DTYPE_E4M3 or TE_DTYPE_E5M2 (got %d, %d)", fn, (int)da, (int)db);
    if (M < 1 || N < 1 || M >= kMaxDim || N >= kMaxDim)
        return fail(TE_ERR_INVALID_ARGUMENT, "%s: M and N must be in [1, 2^31) (got M=%lld N=%lld)", fn, (long long)M, (long long)N);
    if (K < 128 || K % 128 != 0 || K > kMaxK)
        return fail(TE_ERR_INVALID_ARGUMENT, "%s: K must be a positive multiple of 128 up to 2^22 (got %lld)", fn, (long long)K);
    if (accum != TE_ACCUM_FULL_FP32 && accum != TE_ACCUM_FAST)
        return fail(TE_ERR_INVALID_ARGUMENT, "%s: accum must be TE_ACCUM_FULL_FP32 or TE_ACCUM_FAST (got %d)", fn, (int)accum);
    if (!aligned(a, 16) || !aligned(b, 16)) return fail(TE_ERR_MISALIGNED, "%s: fp8 operands must be 16-byte aligned", fn);
    if (!aligned(sa, 16) || !aligned(sb, 16)) return fail(TE_ERR_MISALIGNED, "%s: scales must be 16-byte aligned", fn);
    return TE_OK;
}

// Output matrix [M][ld] of dtype d (bf16 or fp32), base 16-byte aligned, rows 16-byte multiples.
te_status_t check_output(const char* fn, const char* what, const void* p, te_dtype_t d, int64_t ld, int64_t N)
{
    if (!p) return fail(TE_ERR_INVALID_ARGUMENT, "%s: %s pointer is null", fn, what);
    if (d != TE_DTYPE_BF16 && d != TE_DTYPE_F32)
        return fail(TE_ERR_INVALID_ARGUMENT, "%s: %s dtype must be TE_DTYPE_BF16 or TE_DTYPE_F32 (got %d)", fn, what, (int)d);
    if (ld < N) return fail(TE_ERR_INVALID_ARGUMENT, "%s: leading dimension of %s (%lld) is below N (%lld)", fn, what, (long long)ld, (long long)N);
    const int64_t per16 = d == TE_DTYPE_BF16 ? 8 : 4;
    if (!aligned(p, 16) || ld % per16 != 0)
        return fail(TE_ERR_MISALIGNED, "%s: %s must be 16-byte aligned with a row stride that is a multiple of 16 bytes", fn, what);
    return TE_OK;
}

tefp8::GemmArgs base_args(const void* a, const float* sa, te_dtype_t da, const void* b, const float* sb,
                          te_dtype_t db, int64_t M, int64_t N, int64_t K, te_accum_t accum)
{
    tefp8::GemmArgs g;
    std::memset(&g, 0, sizeof g);
    g.a = static_cast<const uint8_t*>(a);
    g.sa = sa;
    g.b = static_cast<const uint8_t*>(b);
    g.sb = sb;
    g.M = M;
    g.N = N;
    g.lda = K;
    g.ldb = K;
    g.lsa = te_scale_ld(M);
    g.lsb = te_scale_ld(N);
    g.fmt_a = to_fmt(da);
    g.fmt_b = to_fmt(db);
    g.fast = accum == TE_ACCUM_FAST;
    g.num_groups = 1;
    g.groups[0] = tefp8::Group{0, (int32_t)(K / 128), 0, 0};
    return g;
}

te_status_t launch(const char* fn, const tefp8::GemmArgs& g, hipStream_t stream, int64_t K, te_dtype_t da,
                   te_dtype_t db, te_accum_t accum, uint32_t epi)
{
    tefp8::LaunchInfo info{};
    hipError_t e = tefp8::launch_gemm(g, stream, &info);
    if (log_enabled())
        std::fprintf(stderr, "[te_fp8] %s M=%lld N=%lld K=%lld a=%s b=%s accum=%s epi=0x%x tile=%dx%d threads=%d grid=%lld groups=%d\n",
                     fn, (long long)g.M, (long long)g.N, (long long)K, dtype_name(da), dtype_name(db),
                     accum == TE_ACCUM_FAST ? "fast" : "full", epi, info.tile_m, info.tile_n, info.threads,
                     (long long)info.grid, g.num_groups);
    if (e != hipSuccess) return fail(TE_ERR_HIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

const char* te_status_string(te_status_t s)
{
    switch (s) {
    case TE_OK: return "TE_OK";
    case TE_ERR_INVALID_ARGUMENT: return "TE_ERR_INVALID_ARGUMENT";
    case TE_ERR_MISALIGNED: return "TE_ERR_MISALIGNED";
    case TE_ERR_UNSUPPORTED: return "TE_ERR_UNSUPPORTED";
    case TE_ERR_HIP: return "TE_ERR_HIP";
    case TE_ERR_INTERNAL: return "TE_ERR_INTERNAL";
    }
    return "TE_ERR_UNKNOWN";
}

const char* te_last_error_message(void) { return g_last_error.c_str(); }

int64_t te_scale_ld(int64_t rows) { return rows > 0 ? (rows + 3) / 4 * 4 : 0; }

namespace {
// The checks of one cast operand (shared by the single and batched casts).
te_status_t check_cast_operand(const char* fn, const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                               const void* q, int64_t ld_q, const float* scales)
{
    if (!x_bf16 || !q || !scales) return fail(TE_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
    if (rows < 1 || rows >= kMaxDim) return fail(TE_ERR_INVALID_ARGUMENT, "%s: rows must be in [1, 2^31) (got %lld)", fn, (long long)rows);
    if (cols < 128 || cols % 128 != 0 || cols >= kMaxDim)
        return fail(TE_ERR_INVALID_ARGUMENT, "%s: cols must be a positive multiple of 128 (got %lld)", fn, (long long)cols);
    if (ld_x < cols || ld_q < cols) return fail(TE_ERR_INVALID_ARGUMENT, "%s: ld_x and ld_q must be >= cols", fn);
    if (!aligned(x_bf16, 16) || ld_x % 8 != 0) return fail(TE_ERR_MISALIGNED, "%s: x must be 16-byte aligned with ld_x a multiple of 8", fn);
    if (!aligned(q, 16) || ld_q % 16 != 0) return fail(TE_ERR_MISALIGNED, "%s: q must be 16-byte aligned with ld_q a multiple of 16", fn);
    if (!aligned(scales, 16)) return fail(TE_ERR_MISALIGNED, "%s: scales must be 16-byte aligned", fn);
    return TE_OK;
}
}  // namespace

te_status_t te_cast_fp8_per_token_batch(const te_cast_operand_t* ops, int32_t n, te_dtype_t out_dtype,
                                        uint32_t flags, hipStream_t stream)
{
    try {
        const char* fn = "te_cast_fp8_per_token_batch";
        if (!ops) return fail(TE_ERR_INVALID_ARGUMENT, "%s: ops is null", fn);
        if (n < 1 || n > tefp8::kMaxCastBatch)
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: n must be in [1, %d] (got %d)", fn, tefp8::kMaxCastBatch, (int)n);
        if (!is_fp8(out_dtype)) return fail(TE_ERR_INVALID_ARGUMENT, "%s: out_dtype must be TE_DTYPE_E4M3 or TE_DTYPE_E5M2 (got %d)", fn, (int)out_dtype);
        if (flags & ~(uint32_t)TE_CAST_POW2_SCALE) return fail(TE_ERR_INVALID_ARGUMENT, "%s: unknown flag bits 0x%x", fn, flags);
        tefp8::CastOperand co[tefp8::kMaxCastBatch] = {};
        for (int32_t i = 0; i < n; ++i) {
            const te_cast_operand_t& o = ops[i];
            te_status_t st = check_cast_operand(fn, o.x_bf16, o.rows, o.cols, o.ld_x, o.q, o.ld_q, o.scales);
            if (st != TE_OK) return fail(st, "%s (operand %d)", te_last_error_message(), (int)i);
            co[i].x = static_cast<const uint16_t*>(o.x_bf16);
            co[i].rows = o.rows;
            co[i].cols = o.cols;
            co[i].ld_x = o.ld_x;
            co[i].q = static_cast<uint8_t*>(o.q);
            co[i].ld_q = o.ld_q;
            co[i].scales = o.scales;
            co[i].ld_s = te_scale_ld(o.rows);
        }
        tefp8::LaunchInfo info{};
        hipError_t e = tefp8::launch_cast_batch(co, n, to_fmt(out_dtype), (flags & TE_CAST_POW2_SCALE) != 0, stream, &info);
        if (log_enabled())
            std::fprintf(stderr, "[te_fp8] %s n=%d out=%s pow2=%d threads=%d grid=%lld\n", fn, (int)n,
                         dtype_name(out_dtype), (flags & TE_CAST_POW2_SCALE) ? 1 : 0, info.threads, (long long)info.grid);
        if (e != hipSuccess) return fail(TE_ERR_HIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
        return ok();
    } catch (...) {
        return fail(TE_ERR_INTERNAL, "te_cast_fp8_per_token_batch: internal error");
    }
}

te_status_t te_cast_fp8_per_token(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                  te_dtype_t out_dtype, uint32_t flags, void* q, int64_t ld_q,
                                  float* scales, hipStream_t stream)
{
    try {
        const char* fn = "te_cast_fp8_per_token";
        if (!x_bf16 || !q || !scales) return fail(TE_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
        if (rows < 1 || rows >= kMaxDim) return fail(TE_ERR_INVALID_ARGUMENT, "%s: rows must be in [1, 2^31) (got %lld)", fn, (long long)rows);
        if (cols < 128 || cols % 128 != 0 || cols >= kMaxDim)
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: cols must be a positive multiple of 128 (got %lld)", fn, (long long)cols);
        if (ld_x < cols || ld_q < cols) return fail(TE_ERR_INVALID_ARGUMENT, "%s: ld_x and ld_q must be >= cols", fn);
        if (!is_fp8(out_dtype)) return fail(TE_ERR_INVALID_ARGUMENT, "%s: out_dtype must be TE_DTYPE_E4M3 or TE_DTYPE_E5M2 (got %d)", fn, (int)out_dtype);
        if (flags & ~(uint32_t)TE_CAST_POW2_SCALE) return fail(TE_ERR_INVALID_ARGUMENT, "%s: unknown flag bits 0x%x", fn, flags);
        if (!aligned(x_bf16, 16) || ld_x % 8 != 0) return fail(TE_ERR_MISALIGNED, "%s: x must be 16-byte aligned with ld_x a multiple of 8", fn);
        if (!aligned(q, 16) || ld_q % 16 != 0) return fail(TE_ERR_MISALIGNED, "%s: q must be 16-byte aligned with ld_q a multiple of 16", fn);
        if (!aligned(scales, 16)) return fail(TE_ERR_MISALIGNED, "%s: scales must be 16-byte aligned", fn);
        tefp8::LaunchInfo info{};
        hipError_t e = tefp8::launch_cast(static_cast<const uint16_t*>(x_bf16), rows, cols, ld_x, to_fmt(out_dtype),
                                          (flags & TE_CAST_POW2_SCALE) != 0, static_cast<uint8_t*>(q), ld_q, scales,
                                          te_scale_ld(rows), stream, &info);
        if (log_enabled())
            std::fprintf(stderr, "[te_fp8] %s rows=%lld cols=%lld out=%s pow2=%d threads=%d grid=%lld\n", fn,
                         (long long)rows, (long long)cols, dtype_name(out_dtype), (flags & TE_CAST_POW2_SCALE) ? 1 : 0,
                         info.threads, (long long)info.grid);
        if (e != hipSuccess) return fail(TE_ERR_HIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
        return ok();
    } catch (...) {
        return fail(TE_ERR_INTERNAL, "te_cast_fp8_per_token: internal error");
    }
}

te_status_t te_cast_fp8_per_token_transpose(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                            te_dtype_t out_dtype, uint32_t flags, void* q, int64_t ld_q,
                                            float* scales, void* qt, int64_t ld_qt, float* scales_t,
                                            hipStream_t stream)
{
    try {
        const char* fn = "te_cast_fp8_per_token_transpose";
        if (!x_bf16 || !qt || !scales_t) return fail(TE_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
        if ((q == nullptr) != (scales == nullptr))
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: q and scales must both be given or both be null", fn);
        if (rows < 128 || rows % 128 != 0 || rows >= kMaxDim)
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: rows must be a positive multiple of 128 (got %lld)", fn, (long long)rows);
        if (q && (cols < 128 || cols % 128 != 0 || cols >= kMaxDim))
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: with the row-wise cast, cols must be a positive multiple of 128 (got %lld)",
                        fn, (long long)cols);
        if (!q && (cols < 8 || cols % 8 != 0 || cols >= kMaxDim))
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: cols must be a positive multiple of 8 (got %lld)", fn, (long long)cols);
        if (ld_x < cols || (q && ld_q < cols) || ld_qt < rows)
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: ld_x and ld_q must be >= cols, ld_qt >= rows", fn);
        if (!is_fp8(out_dtype)) return fail(TE_ERR_INVALID_ARGUMENT, "%s: out_dtype must be TE_DTYPE_E4M3 or TE_DTYPE_E5M2 (got %d)", fn, (int)out_dtype);
        if (flags & ~(uint32_t)TE_CAST_POW2_SCALE) return fail(TE_ERR_INVALID_ARGUMENT, "%s: unknown flag bits 0x%x", fn, flags);
        if (!aligned(x_bf16, 16) || ld_x % 8 != 0) return fail(TE_ERR_MISALIGNED, "%s: x must be 16-byte aligned with ld_x a multiple of 8", fn);
        if (q && (!aligned(q, 16) || ld_q % 16 != 0)) return fail(TE_ERR_MISALIGNED, "%s: q must be 16-byte aligned with ld_q a multiple of 16", fn);
        if (!aligned(qt, 16) || ld_qt % 16 != 0) return fail(TE_ERR_MISALIGNED, "%s: qt must be 16-byte aligned with ld_qt a multiple of 16", fn);
        if ((scales && !aligned(scales, 16)) || !aligned(scales_t, 16))
            return fail(TE_ERR_MISALIGNED, "%s: scales and scales_t must be 16-byte aligned", fn);
        tefp8::LaunchInfo info{};
        hipError_t e = tefp8::launch_cast_transpose(
            static_cast<const uint16_t*>(x_bf16), rows, cols, ld_x, to_fmt(out_dtype), (flags & TE_CAST_POW2_SCALE) != 0,
            static_cast<uint8_t*>(q), ld_q, scales, te_scale_ld(rows), static_cast<uint8_t*>(qt), ld_qt, scales_t,
            te_scale_ld(cols), stream, &info);
        if (log_enabled())
            std::fprintf(stderr, "[te_fp8] %s rows=%lld cols=%lld out=%s pow2=%d rowwise=%d threads=%d grid=%lld\n", fn,
                         (long long)rows, (long long)cols, dtype_name(out_dtype), (flags & TE_CAST_POW2_SCALE) ? 1 : 0,
                         q ? 1 : 0, info.threads, (long long)info.grid);
        if (e != hipSuccess) return fail(TE_ERR_HIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
        return ok();
    } catch (...) {
        return fail(TE_ERR_INTERNAL, "te_cast_fp8_per_token_transpose: internal error");
    }
}

te_status_t te_fp8_gemm_fwd(const void* x, const float* x_scales, te_dtype_t x_dtype,
                            const void* w, const float* w_scales, te_dtype_t w_dtype,
                            int64_t M, int64_t N, int64_t K,
                            const void* bias_bf16, uint32_t epilogue,
                            void* y, te_dtype_t y_dtype, int64_t ld_y,
                            void* preact_bf16, int64_t ld_preact,
                            te_accum_t accum, hipStream_t stream)
{
    try {
        const char* fn = "te_fp8_gemm_fwd";
        te_status_t st = check_operands(fn, x, x_scales, x_dtype, w, w_scales, w_dtype, M, N, K, accum);
        if (st != TE_OK) return st;
        const uint32_t allowed = TE_EPI_BIAS | TE_EPI_GELU | TE_EPI_AUX_PREACT;
        if (epilogue & ~allowed) return fail(TE_ERR_INVALID_ARGUMENT, "%s: epilogue flags 0x%x are not forward flags", fn, epilogue);
        if ((epilogue & TE_EPI_AUX_PREACT) && !(epilogue & TE_EPI_GELU))
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: TE_EPI_AUX_PREACT requires TE_EPI_GELU", fn);
        if ((epilogue & TE_EPI_BIAS) && !bias_bf16) return fail(TE_ERR_INVALID_ARGUMENT, "%s: TE_EPI_BIAS needs bias_bf16", fn);
        if (bias_bf16 && !(epilogue & TE_EPI_BIAS)) return fail(TE_ERR_INVALID_ARGUMENT, "%s: bias_bf16 given without TE_EPI_BIAS", fn);
        if (bias_bf16 && !aligned(bias_bf16, 16)) return fail(TE_ERR_MISALIGNED, "%s: bias must be 16-byte aligned", fn);
        st = check_output(fn, "y", y, y_dtype, ld_y, N);
        if (st != TE_OK) return st;
        if (epilogue & TE_EPI_AUX_PREACT) {
            st = check_output(fn, "preact", preact_bf16, TE_DTYPE_BF16, ld_preact, N);
            if (st != TE_OK) return st;
        } else if (preact_bf16) {
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: preact given without TE_EPI_AUX_PREACT", fn);
        }
        tefp8::GemmArgs g = base_args(x, x_scales, x_dtype, w, w_scales, w_dtype, M, N, K, accum);
        g.epi = tefp8::Epi::Fwd;
        g.flags = epilogue;
        g.out = y;
        g.out_bf16 = y_dtype == TE_DTYPE_BF16;
        g.ld_out = ld_y;
        g.bias = static_cast<const uint16_t*>(bias_bf16);
        g.aux = static_cast<uint16_t*>(preact_bf16);
        g.ld_aux = ld_preact;
        return launch(fn, g, stream, K, x_dtype, w_dtype, accum, epilogue);
    } catch (...) {
        return fail(TE_ERR_INTERNAL, "te_fp8_gemm_fwd: internal error");
    }
}

te_status_t te_fp8_gemm_dgrad(const void* dy, const float* dy_scales, te_dtype_t dy_dtype,
                              const void* wt, const float* wt_scales, te_dtype_t wt_dtype,
                              int64_t M, int64_t N, int64_t K, uint32_t epilogue,
                              const void* preact_bf16, int64_t ld_preact,
                              float* bias_grad,
                              void* dx, te_dtype_t dx_dtype, int64_t ld_dx,
                              te_accum_t accum, hipStream_t stream)
{
    try {
        const char* fn = "te_fp8_gemm_dgrad";
        te_status_t st = check_operands(fn, dy, dy_scales, dy_dtype, wt, wt_scales, wt_dtype, M, N, K, accum);
        if (st != TE_OK) return st;
        const uint32_t allowed = TE_EPI_DGELU | TE_EPI_BGRAD;
        if (epilogue & ~allowed) return fail(TE_ERR_INVALID_ARGUMENT, "%s: epilogue flags 0x%x are not dgrad flags", fn, epilogue);
        if (epilogue & TE_EPI_DGELU) {
            if (!preact_bf16) return fail(TE_ERR_INVALID_ARGUMENT, "%s: TE_EPI_DGELU needs preact_bf16", fn);
            if (ld_preact < N) return fail(TE_ERR_INVALID_ARGUMENT, "%s: ld_preact (%lld) is below N", fn, (long long)ld_preact);
            if (!aligned(preact_bf16, 16) || ld_preact % 8 != 0)
                return fail(TE_ERR_MISALIGNED, "%s: preact must be 16-byte aligned with ld_preact a multiple of 8", fn);
        } else if (preact_bf16) {
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: preact given without TE_EPI_DGELU", fn);
        }
        if (epilogue & TE_EPI_BGRAD) {
            if (!bias_grad) return fail(TE_ERR_INVALID_ARGUMENT, "%s: TE_EPI_BGRAD needs bias_grad", fn);
            if (!aligned(bias_grad, 4)) return fail(TE_ERR_MISALIGNED, "%s: bias_grad must be 4-byte aligned", fn);
        } else if (bias_grad) {
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: bias_grad given without TE_EPI_BGRAD", fn);
        }
        st = check_output(fn, "dx", dx, dx_dtype, ld_dx, N);
        if (st != TE_OK) return st;
        tefp8::GemmArgs g = base_args(dy, dy_scales, dy_dtype, wt, wt_scales, wt_dtype, M, N, K, accum);
        g.epi = tefp8::Epi::Dgrad;
        g.flags = epilogue;
        g.out = dx;
        g.out_bf16 = dx_dtype == TE_DTYPE_BF16;
        g.ld_out = ld_dx;
        g.preact = static_cast<const uint16_t*>(preact_bf16);
        g.ld_aux = ld_preact;
        g.bias_grad = bias_grad;
        if (epilogue & TE_EPI_BGRAD) {
            hipError_t e = tefp8::launch_zero_f32(bias_grad, N, stream);
            if (e != hipSuccess) return fail(TE_ERR_HIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
        }
        return launch(fn, g, stream, K, dy_dtype, wt_dtype, accum, epilogue);
    } catch (...) {
        return fail(TE_ERR_INTERNAL, "te_fp8_gemm_dgrad: internal error");
    }
}

te_status_t te_fp8_wgrad_accum(const void* a, const float* a_scales, te_dtype_t a_dtype,
                               const void* b, const float* b_scales, te_dtype_t b_dtype,
                               int64_t M, int64_t N, int64_t K,
                               float* out, int64_t ld_out,
                               te_accum_t accum, hipStream_t stream)
{
    try {
        const char* fn = "te_fp8_wgrad_accum";
        te_status_t st = check_operands(fn, a, a_scales, a_dtype, b, b_scales, b_dtype, M, N, K, accum);
        if (st != TE_OK) return st;
        st = check_output(fn, "out", out, TE_DTYPE_F32, ld_out, N);
        if (st != TE_OK) return st;
        tefp8::GemmArgs g = base_args(a, a_scales, a_dtype, b, b_scales, b_dtype, M, N, K, accum);
        g.epi = tefp8::Epi::Wgrad;
        g.out = out;
        g.ld_out = ld_out;
        return launch(fn, g, stream, K, a_dtype, b_dtype, accum, 0);
    } catch (...) {
        return fail(TE_ERR_INTERNAL, "te_fp8_wgrad_accum: internal error");
    }
}

te_status_t te_fp8_wgrad_accum_bgrad(const void* a, const float* a_scales, te_dtype_t a_dtype,
                                     const void* b, const float* b_scales, te_dtype_t b_dtype,
                                     int64_t M, int64_t N, int64_t K,
                                     float* out, int64_t ld_out, float* bias_grad,
                                     te_accum_t accum, hipStream_t stream)
{
    try {
        const char* fn = "te_fp8_wgrad_accum_bgrad";
        te_status_t st = check_operands(fn, a, a_scales, a_dtype, b, b_scales, b_dtype, M, N, K, accum);
        if (st != TE_OK) return st;
        st = check_output(fn, "out", out, TE_DTYPE_F32, ld_out, N);
        if (st != TE_OK) return st;
        if (!bias_grad) return fail(TE_ERR_INVALID_ARGUMENT, "%s: bias_grad is null", fn);
        if (!aligned(bias_grad, 4)) return fail(TE_ERR_MISALIGNED, "%s: bias_grad must be 4-byte aligned", fn);
        tefp8::GemmArgs g = base_args(a, a_scales, a_dtype, b, b_scales, b_dtype, M, N, K, accum);
        g.epi = tefp8::Epi::Wgrad;
        g.out = out;
        g.ld_out = ld_out;
        st = launch(fn, g, stream, K, a_dtype, b_dtype, accum, 0);
        if (st != TE_OK) return st;
        hipError_t e = tefp8::launch_row_sum(static_cast<const uint8_t*>(a), M, K, K, to_fmt(a_dtype), a_scales,
                                             te_scale_ld(M), bias_grad, stream);
        if (e != hipSuccess) return fail(TE_ERR_HIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
        return ok();
    } catch (...) {
        return fail(TE_ERR_INTERNAL, "te_fp8_wgrad_accum_bgrad: internal error");
    }
}

te_status_t te_fp8_kgrouped_wgrad(const void* a, const float* a_scales, te_dtype_t a_dtype,
                                  const void* b, const float* b_scales, te_dtype_t b_dtype,
                                  int64_t M, int64_t N, const int64_t* group_k, int32_t G,
                                  float* out, te_accum_t accum, hipStream_t stream)
{
    try {
        const char* fn = "te_fp8_kgrouped_wgrad";
        if (!group_k) return fail(TE_ERR_INVALID_ARGUMENT, "%s: group_k is null", fn);
        if (G < 1 || G > 1024) return fail(TE_ERR_INVALID_ARGUMENT, "%s: G must be in [1, 1024] (got %d)", fn, (int)G);
        int64_t sumk = 0;
        for (int32_t g = 0; g < G; ++g) {
            if (group_k[g] < 0 || group_k[g] % 128 != 0 || group_k[g] > kMaxK)
                return fail(TE_ERR_INVALID_ARGUMENT, "%s: group_k[%d] = %lld is not a non-negative multiple of 128", fn, (int)g,
                            (long long)group_k[g]);
            sumk += group_k[g];
        }
        te_status_t st = check_operands(fn, a, a_scales, a_dtype, b, b_scales, b_dtype, M, N, sumk, accum);
        if (st != TE_OK) return st;
        st = check_output(fn, "out", out, TE_DTYPE_F32, N, N);
        if (st != TE_OK) return st;

        // longest group first; empty groups get no work
        std::vector<tefp8::Group> work;
        int64_t off = 0;
        for (int32_t g = 0; g < G; ++g) {
            if (group_k[g] > 0) work.push_back(tefp8::Group{(int32_t)(off / 128), (int32_t)(group_k[g] / 128), g, 0});
            off += group_k[g];
        }
        std::stable_sort(work.begin(), work.end(),
                         [](const tefp8::Group& x, const tefp8::Group& y) { return x.kb_len > y.kb_len; });

        tefp8::GemmArgs g = base_args(a, a_scales, a_dtype, b, b_scales, b_dtype, M, N, sumk, accum);
        g.epi = tefp8::Epi::Wgrad;
        g.out = out;
        g.ld_out = N;
        g.out_group_stride = M * N;
        for (size_t start = 0; start < work.size(); start += tefp8::kMaxGroupsPerLaunch) {
            const size_t cnt = std::min(work.size() - start, (size_t)tefp8::kMaxGroupsPerLaunch);
            g.num_groups = (int)cnt;
            for (size_t i = 0; i < cnt; ++i) g.groups[i] = work[start + i];
            st = launch(fn, g, stream, sumk, a_dtype, b_dtype, accum, 0);
            if (st != TE_OK) return st;
        }
        return ok();
    } catch (...) {
        return fail(TE_ERR_INTERNAL, "te_fp8_kgrouped_wgrad: internal error");
    }
}

te_status_t te_fp8_kgrouped_wgrad_device_sizes(const void* a, const float* a_scales, te_dtype_t a_dtype,
                                               const void* b, const float* b_scales, te_dtype_t b_dtype,
                                               int64_t M, int64_t N, int64_t sum_k, const int64_t* group_k_device,
                                               int32_t G, float* out, te_accum_t accum, hipStream_t stream)
{
    try {
        const char* fn = "te_fp8_kgrouped_wgrad_device_sizes";
        if (!group_k_device) return fail(TE_ERR_INVALID_ARGUMENT, "%s: group_k_device is null", fn);
        if (!aligned(group_k_device, 8)) return fail(TE_ERR_MISALIGNED, "%s: group_k_device must be 8-byte aligned", fn);
        if (G < 1 || G > tefp8::kMaxDeviceGroups)
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: G must be in [1, %d] (got %d)", fn, tefp8::kMaxDeviceGroups, (int)G);
        te_status_t st = check_operands(fn, a, a_scales, a_dtype, b, b_scales, b_dtype, M, N, sum_k, accum);
        if (st != TE_OK) return st;
        st = check_output(fn, "out", out, TE_DTYPE_F32, N, N);
        if (st != TE_OK) return st;
        tefp8::GemmArgs g = base_args(a, a_scales, a_dtype, b, b_scales, b_dtype, M, N, sum_k, accum);
        g.epi = tefp8::Epi::Wgrad;
        g.out = out;
        g.ld_out = N;
        g.out_group_stride = M * N;
        g.num_groups = G;
        g.group_k_dev = group_k_device;
        g.sum_kb = sum_k / 128;
        return launch(fn, g, stream, sum_k, a_dtype, b_dtype, accum, 0);
    } catch (...) {
        return fail(TE_ERR_INTERNAL, "te_fp8_kgrouped_wgrad_device_sizes: internal error");
    }
}

te_status_t te_fp8_mgrouped_gemm_fwd(const void* x, const float* x_scales, te_dtype_t x_dtype,
                                     const void* w, const float* w_scales, te_dtype_t w_dtype,
                                     int64_t sum_m, int64_t N, int64_t K, int32_t G, const int32_t* m_block_group,
                                     const void* bias_bf16, uint32_t epilogue,
                                     void* y, te_dtype_t y_dtype, int64_t ld_y,
                                     void* preact_bf16, int64_t ld_preact,
                                     te_accum_t accum, hipStream_t stream)
{
    try {
        const char* fn = "te_fp8_mgrouped_gemm_fwd";
        if (!m_block_group) return fail(TE_ERR_INVALID_ARGUMENT, "%s: m_block_group is null", fn);
        if (!aligned(m_block_group, 4)) return fail(TE_ERR_MISALIGNED, "%s: m_block_group must be 4-byte aligned", fn);
        if (G < 1 || G > 1024) return fail(TE_ERR_INVALID_ARGUMENT, "%s: G must be in [1, 1024] (got %d)", fn, (int)G);
        if (sum_m < tefp8::kMGroupRows || sum_m % tefp8::kMGroupRows != 0)
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: sum_m must be a positive multiple of %d (got %lld)", fn,
                        tefp8::kMGroupRows, (long long)sum_m);
        te_status_t st = check_operands(fn, x, x_scales, x_dtype, w, w_scales, w_dtype, sum_m, N, K, accum);
        if (st != TE_OK) return st;
        const uint32_t allowed = TE_EPI_BIAS | TE_EPI_GELU | TE_EPI_AUX_PREACT;
        if (epilogue & ~allowed) return fail(TE_ERR_INVALID_ARGUMENT, "%s: epilogue 0x%x has flags other than BIAS|GELU|AUX_PREACT", fn, epilogue);
        if ((epilogue & TE_EPI_AUX_PREACT) && !(epilogue & TE_EPI_GELU))
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: TE_EPI_AUX_PREACT needs TE_EPI_GELU", fn);
        if ((epilogue & TE_EPI_BIAS) && !bias_bf16) return fail(TE_ERR_INVALID_ARGUMENT, "%s: TE_EPI_BIAS needs bias_bf16", fn);
        if (bias_bf16 && !(epilogue & TE_EPI_BIAS)) return fail(TE_ERR_INVALID_ARGUMENT, "%s: bias_bf16 given without TE_EPI_BIAS", fn);
        if (bias_bf16 && !aligned(bias_bf16, 16)) return fail(TE_ERR_MISALIGNED, "%s: bias must be 16-byte aligned", fn);
        if ((epilogue & TE_EPI_BIAS) && N % 8 != 0)
            return fail(TE_ERR_MISALIGNED, "%s: with a bias, N must be a multiple of 8 (each expert's bias row 16-byte aligned)", fn);
        st = check_output(fn, "y", y, y_dtype, ld_y, N);
        if (st != TE_OK) return st;
        if (epilogue & TE_EPI_AUX_PREACT) {
            st = check_output(fn, "preact", preact_bf16, TE_DTYPE_BF16, ld_preact, N);
            if (st != TE_OK) return st;
        } else if (preact_bf16) {
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: preact given without TE_EPI_AUX_PREACT", fn);
        }
        tefp8::GemmArgs g = base_args(x, x_scales, x_dtype, w, w_scales, w_dtype, sum_m, N, K, accum);
        g.epi = tefp8::Epi::Fwd;
        g.flags = epilogue;
        g.out = y;
        g.out_bf16 = y_dtype == TE_DTYPE_BF16;
        g.ld_out = ld_y;
        g.bias = static_cast<const uint16_t*>(bias_bf16);
        g.aux = static_cast<uint16_t*>(preact_bf16);
        g.ld_aux = ld_preact;
        g.m_block_group = m_block_group;
        g.num_b_groups = G;
        g.b_group_stride = N * K;
        g.sb_group_stride = (K / 128) * te_scale_ld(N);
        g.bias_group_stride = N;
        return launch(fn, g, stream, K, x_dtype, w_dtype, accum, epilogue);
    } catch (...) {
        return fail(TE_ERR_INTERNAL, "te_fp8_mgrouped_gemm_fwd: internal error");
    }
}

// The quantised outputs of the quantising GEMMs: the row-wise cast (q, q_scales) and/or the cast
// of the transpose (qt, qt_scales); at least one pair.
static te_status_t check_quant_outputs(const char* fn, int64_t M, int64_t N, const void* q, int64_t ld_q,
                                       const float* q_scales, const void* qt, int64_t ld_qt, const float* qt_scales)
{
    if (!q && !qt) return fail(TE_ERR_INVALID_ARGUMENT, "%s: q or qt (or both) is required", fn);
    if (q || q_scales) {
        if (!q || !q_scales) return fail(TE_ERR_INVALID_ARGUMENT, "%s: q and q_scales go together", fn);
        if (ld_q < N) return fail(TE_ERR_INVALID_ARGUMENT, "%s: ld_q must be >= N", fn);
        if (!aligned(q, 16) || ld_q % 16 != 0)
            return fail(TE_ERR_MISALIGNED, "%s: q must be 16-byte aligned with ld_q a multiple of 16", fn);
        if (!aligned(q_scales, 16)) return fail(TE_ERR_MISALIGNED, "%s: q_scales must be 16-byte aligned", fn);
    }
    if (qt || qt_scales) {
        if (!qt || !qt_scales) return fail(TE_ERR_INVALID_ARGUMENT, "%s: qt and qt_scales go together", fn);
        if (M % 128 != 0)
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: the transposed cast needs M a multiple of 128 (got %lld)", fn,
                        (long long)M);
        if (ld_qt < M) return fail(TE_ERR_INVALID_ARGUMENT, "%s: ld_qt must be >= M", fn);
        if (!aligned(qt, 16) || ld_qt % 16 != 0)
            return fail(TE_ERR_MISALIGNED, "%s: qt must be 16-byte aligned with ld_qt a multiple of 16", fn);
        if (!aligned(qt_scales, 16)) return fail(TE_ERR_MISALIGNED, "%s: qt_scales must be 16-byte aligned", fn);
    }
    return TE_OK;
}

te_status_t te_fp8_gemm_fwd_quant(const void* x, const float* x_scales, te_dtype_t x_dtype,
                                  const void* w, const float* w_scales, te_dtype_t w_dtype,
                                  int64_t M, int64_t N, int64_t K,
                                  const void* bias_bf16, uint32_t epilogue,
                                  te_dtype_t q_dtype, uint32_t cast_flags, void* q, int64_t ld_q, float* q_scales,
                                  void* qt, int64_t ld_qt, float* qt_scales,
                                  void* preact_bf16, int64_t ld_preact,
                                  te_accum_t accum, hipStream_t stream)
{
    try {
        const char* fn = "te_fp8_gemm_fwd_quant";
        te_status_t st = check_operands(fn, x, x_scales, x_dtype, w, w_scales, w_dtype, M, N, K, accum);
        if (st != TE_OK) return st;
        if (N % 128 != 0) return fail(TE_ERR_INVALID_ARGUMENT, "%s: N must be a multiple of 128 (whole 1x128 groups; got %lld)", fn, (long long)N);
        const uint32_t allowed = TE_EPI_BIAS | TE_EPI_GELU | TE_EPI_AUX_PREACT;
        if (epilogue & ~allowed) return fail(TE_ERR_INVALID_ARGUMENT, "%s: epilogue flags 0x%x are not forward flags", fn, epilogue);
        if ((epilogue & TE_EPI_AUX_PREACT) && !(epilogue & TE_EPI_GELU))
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: TE_EPI_AUX_PREACT requires TE_EPI_GELU", fn);
        if ((epilogue & TE_EPI_BIAS) && !bias_bf16) return fail(TE_ERR_INVALID_ARGUMENT, "%s: TE_EPI_BIAS needs bias_bf16", fn);
        if (bias_bf16 && !(epilogue & TE_EPI_BIAS)) return fail(TE_ERR_INVALID_ARGUMENT, "%s: bias_bf16 given without TE_EPI_BIAS", fn);
        if (bias_bf16 && !aligned(bias_bf16, 16)) return fail(TE_ERR_MISALIGNED, "%s: bias must be 16-byte aligned", fn);
        if (!is_fp8(q_dtype)) return fail(TE_ERR_INVALID_ARGUMENT, "%s: q_dtype must be TE_DTYPE_E4M3 or TE_DTYPE_E5M2 (got %d)", fn, (int)q_dtype);
        if (cast_flags & ~(uint32_t)TE_CAST_POW2_SCALE) return fail(TE_ERR_INVALID_ARGUMENT, "%s: unknown cast flag bits 0x%x", fn, cast_flags);
        st = check_quant_outputs(fn, M, N, q, ld_q, q_scales, qt, ld_qt, qt_scales);
        if (st != TE_OK) return st;
        if (epilogue & TE_EPI_AUX_PREACT) {
            st = check_output(fn, "preact", preact_bf16, TE_DTYPE_BF16, ld_preact, N);
            if (st != TE_OK) return st;
        } else if (preact_bf16) {
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: preact given without TE_EPI_AUX_PREACT", fn);
        }
        tefp8::GemmArgs g = base_args(x, x_scales, x_dtype, w, w_scales, w_dtype, M, N, K, accum);
        g.epi = tefp8::Epi::Fwd;
        g.flags = epilogue;
        g.bias = static_cast<const uint16_t*>(bias_bf16);
        g.aux = static_cast<uint16_t*>(preact_bf16);
        g.ld_aux = ld_preact;
        g.q_out = static_cast<uint8_t*>(q);
        g.q_scales = q_scales;
        g.ld_q = ld_q;
        g.ld_qs = te_scale_ld(M);
        g.q_fmt = to_fmt(q_dtype);
        g.q_pow2 = (cast_flags & TE_CAST_POW2_SCALE) ? 1 : 0;
        g.qt_out = static_cast<uint8_t*>(qt);
        g.qt_scales = qt_scales;
        g.ld_qt = ld_qt;
        g.ld_qts = te_scale_ld(N);
        return launch(fn, g, stream, K, x_dtype, w_dtype, accum, epilogue);
    } catch (...) {
        return fail(TE_ERR_INTERNAL, "te_fp8_gemm_fwd_quant: internal error");
    }
}

te_status_t te_fp8_gemm_dgrad_quant(const void* dy, const float* dy_scales, te_dtype_t dy_dtype,
                                    const void* wt, const float* wt_scales, te_dtype_t wt_dtype,
                                    int64_t M, int64_t N, int64_t K, uint32_t epilogue,
                                    const void* preact_bf16, int64_t ld_preact, float* bias_grad,
                                    te_dtype_t q_dtype, uint32_t cast_flags, void* q, int64_t ld_q, float* q_scales,
                                    void* qt, int64_t ld_qt, float* qt_scales,
                                    te_accum_t accum, hipStream_t stream)
{
    try {
        const char* fn = "te_fp8_gemm_dgrad_quant";
        te_status_t st = check_operands(fn, dy, dy_scales, dy_dtype, wt, wt_scales, wt_dtype, M, N, K, accum);
        if (st != TE_OK) return st;
        if (N % 128 != 0) return fail(TE_ERR_INVALID_ARGUMENT, "%s: N must be a multiple of 128 (whole 1x128 groups; got %lld)", fn, (long long)N);
        const uint32_t allowed = TE_EPI_DGELU | TE_EPI_BGRAD;
        if (epilogue & ~allowed) return fail(TE_ERR_INVALID_ARGUMENT, "%s: epilogue flags 0x%x are not dgrad flags", fn, epilogue);
        if (epilogue & TE_EPI_DGELU) {
            if (!preact_bf16) return fail(TE_ERR_INVALID_ARGUMENT, "%s: TE_EPI_DGELU needs preact_bf16", fn);
            if (ld_preact < N) return fail(TE_ERR_INVALID_ARGUMENT, "%s: ld_preact (%lld) is below N", fn, (long long)ld_preact);
            if (!aligned(preact_bf16, 16) || ld_preact % 8 != 0)
                return fail(TE_ERR_MISALIGNED, "%s: preact must be 16-byte aligned with ld_preact a multiple of 8", fn);
        } else if (preact_bf16) {
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: preact given without TE_EPI_DGELU", fn);
        }
        if (epilogue & TE_EPI_BGRAD) {
            if (!bias_grad) return fail(TE_ERR_INVALID_ARGUMENT, "%s: TE_EPI_BGRAD needs bias_grad", fn);
            if (!aligned(bias_grad, 4)) return fail(TE_ERR_MISALIGNED, "%s: bias_grad must be 4-byte aligned", fn);
        } else if (bias_grad) {
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: bias_grad given without TE_EPI_BGRAD", fn);
        }
        if (!is_fp8(q_dtype)) return fail(TE_ERR_INVALID_ARGUMENT, "%s: q_dtype must be TE_DTYPE_E4M3 or TE_DTYPE_E5M2 (got %d)", fn, (int)q_dtype);
        if (cast_flags & ~(uint32_t)TE_CAST_POW2_SCALE) return fail(TE_ERR_INVALID_ARGUMENT, "%s: unknown cast flag bits 0x%x", fn, cast_flags);
        st = check_quant_outputs(fn, M, N, q, ld_q, q_scales, qt, ld_qt, qt_scales);
        if (st != TE_OK) return st;
        tefp8::GemmArgs g = base_args(dy, dy_scales, dy_dtype, wt, wt_scales, wt_dtype, M, N, K, accum);
        g.epi = tefp8::Epi::Dgrad;
        g.flags = epilogue;
        g.preact = static_cast<const uint16_t*>(preact_bf16);
        g.ld_aux = ld_preact;
        g.bias_grad = bias_grad;
        g.q_out = static_cast<uint8_t*>(q);
        g.q_scales = q_scales;
        g.ld_q = ld_q;
        g.ld_qs = te_scale_ld(M);
        g.q_fmt = to_fmt(q_dtype);
        g.q_pow2 = (cast_flags & TE_CAST_POW2_SCALE) ? 1 : 0;
        g.qt_out = static_cast<uint8_t*>(qt);
        g.qt_scales = qt_scales;
        g.ld_qt = ld_qt;
        g.ld_qts = te_scale_ld(N);
        if (epilogue & TE_EPI_BGRAD) {
            hipError_t e = tefp8::launch_zero_f32(bias_grad, N, stream);
            if (e != hipSuccess) return fail(TE_ERR_HIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
        }
        return launch(fn, g, stream, K, dy_dtype, wt_dtype, accum, epilogue);
    } catch (...) {
        return fail(TE_ERR_INTERNAL, "te_fp8_gemm_dgrad_quant: internal error");
    }
}

int64_t te_fp8_dgrad_bgrad_workspace_bytes(int64_t M, int64_t N)
{
    if (M < 1 || N < 1) return 0;
    const int64_t rows = (M + 255) / 256 * tefp8::kBgradRowsPerTile;
    return rows * ((N + 3) / 4 * 4) * (int64_t)sizeof(float);
}

// The deterministic dgrad on a given column-sum workspace (caller's or the library's scratch).
static te_status_t dgrad_deterministic(const char* fn, const void* dy, const float* dy_scales, te_dtype_t dy_dtype,
                                       const void* wt, const float* wt_scales, te_dtype_t wt_dtype, int64_t M,
                                       int64_t N, int64_t K, uint32_t epilogue, const void* preact_bf16,
                                       int64_t ld_preact, float* bias_grad, float* ws, void* dx, te_dtype_t dx_dtype,
                                       int64_t ld_dx, te_accum_t accum, hipStream_t stream)
{
    if (!(epilogue & TE_EPI_BGRAD))
        return fail(TE_ERR_INVALID_ARGUMENT, "%s: the epilogue must include TE_EPI_BGRAD", fn);
    te_status_t st = check_operands(fn, dy, dy_scales, dy_dtype, wt, wt_scales, wt_dtype, M, N, K, accum);
    if (st != TE_OK) return st;
    const uint32_t allowed = TE_EPI_DGELU | TE_EPI_BGRAD;
    if (epilogue & ~allowed) return fail(TE_ERR_INVALID_ARGUMENT, "%s: epilogue flags 0x%x are not dgrad flags", fn, epilogue);
    if (epilogue & TE_EPI_DGELU) {
        if (!preact_bf16) return fail(TE_ERR_INVALID_ARGUMENT, "%s: TE_EPI_DGELU needs preact_bf16", fn);
        if (ld_preact < N) return fail(TE_ERR_INVALID_ARGUMENT, "%s: ld_preact (%lld) is below N", fn, (long long)ld_preact);
        if (!aligned(preact_bf16, 16) || ld_preact % 8 != 0)
            return fail(TE_ERR_MISALIGNED, "%s: preact must be 16-byte aligned with ld_preact a multiple of 8", fn);
    } else if (preact_bf16) {
        return fail(TE_ERR_INVALID_ARGUMENT, "%s: preact given without TE_EPI_DGELU", fn);
    }
    if (!bias_grad) return fail(TE_ERR_INVALID_ARGUMENT, "%s: TE_EPI_BGRAD needs bias_grad", fn);
    if (!aligned(bias_grad, 4)) return fail(TE_ERR_MISALIGNED, "%s: bias_grad must be 4-byte aligned", fn);
    st = check_output(fn, "dx", dx, dx_dtype, ld_dx, N);
    if (st != TE_OK) return st;
    if (!ws) {
        // the library's scratch (looked up once per device; no allocation)
        void* p = nullptr;
        hipError_t e = tefp8::noalloc_scratch(&p);
        if (e != hipSuccess) return fail(TE_ERR_HIP, "%s: scratch lookup failed: %s", fn, hipGetErrorString(e));
        ws = static_cast<float*>(p);
    }
    tefp8::GemmArgs g = base_args(dy, dy_scales, dy_dtype, wt, wt_scales, wt_dtype, M, N, K, accum);
    g.epi = tefp8::Epi::Dgrad;
    g.flags = epilogue;
    g.out = dx;
    g.out_bf16 = dx_dtype == TE_DTYPE_BF16;
    g.ld_out = ld_dx;
    g.preact = static_cast<const uint16_t*>(preact_bf16);
    g.ld_aux = ld_preact;
    g.bias_grad = bias_grad;
    g.bgrad_ws = ws;
    g.bgrad_ws_ld = (N + 3) / 4 * 4;
    st = launch(fn, g, stream, K, dy_dtype, wt_dtype, accum, epilogue);
    if (st != TE_OK) return st;
    const int64_t rows = (M + 255) / 256 * tefp8::kBgradRowsPerTile;
    hipError_t e = tefp8::launch_bgrad_reduce(g.bgrad_ws, rows, g.bgrad_ws_ld, N, bias_grad, stream);
    if (e != hipSuccess) return fail(TE_ERR_HIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

te_status_t te_fp8_gemm_dgrad_deterministic(const void* dy, const float* dy_scales, te_dtype_t dy_dtype,
                                            const void* wt, const float* wt_scales, te_dtype_t wt_dtype,
                                            int64_t M, int64_t N, int64_t K, uint32_t epilogue,
                                            const void* preact_bf16, int64_t ld_preact,
                                            float* bias_grad, void* workspace, int64_t workspace_bytes,
                                            void* dx, te_dtype_t dx_dtype, int64_t ld_dx,
                                            te_accum_t accum, hipStream_t stream)
{
    try {
        const char* fn = "te_fp8_gemm_dgrad_deterministic";
        if (!workspace) return fail(TE_ERR_INVALID_ARGUMENT, "%s: workspace is null", fn);
        if (!aligned(workspace, 16)) return fail(TE_ERR_MISALIGNED, "%s: workspace must be 16-byte aligned", fn);
        const int64_t need = te_fp8_dgrad_bgrad_workspace_bytes(M, N);
        if (M >= 1 && N >= 1 && workspace_bytes < need)
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: workspace_bytes %lld below the %lld bytes needed", fn,
                        (long long)workspace_bytes, (long long)need);
        return dgrad_deterministic(fn, dy, dy_scales, dy_dtype, wt, wt_scales, wt_dtype, M, N, K, epilogue,
                                   preact_bf16, ld_preact, bias_grad, static_cast<float*>(workspace), dx, dx_dtype,
                                   ld_dx, accum, stream);
    } catch (...) {
        return fail(TE_ERR_INTERNAL, "te_fp8_gemm_dgrad_deterministic: internal error");
    }
}

te_status_t te_fp8_gemm_dgrad_deterministic_noalloc(const void* dy, const float* dy_scales, te_dtype_t dy_dtype,
                                                    const void* wt, const float* wt_scales, te_dtype_t wt_dtype,
                                                    int64_t M, int64_t N, int64_t K, uint32_t epilogue,
                                                    const void* preact_bf16, int64_t ld_preact, float* bias_grad,
                                                    void* dx, te_dtype_t dx_dtype, int64_t ld_dx,
                                                    te_accum_t accum, hipStream_t stream)
{
    try {
        const char* fn = "te_fp8_gemm_dgrad_deterministic_noalloc";
        const int64_t need = te_fp8_dgrad_bgrad_workspace_bytes(M, N);
        if (need > (int64_t)TE_NOALLOC_SCRATCH_BYTES)
            return fail(TE_ERR_INVALID_ARGUMENT,
                        "%s: an %lld x %lld output needs %lld bytes of column-sum scratch, above the library's "
                        "%lld-byte static array; use te_fp8_gemm_dgrad_deterministic with a workspace",
                        fn, (long long)M, (long long)N, (long long)need, (long long)TE_NOALLOC_SCRATCH_BYTES);
        return dgrad_deterministic(fn, dy, dy_scales, dy_dtype, wt, wt_scales, wt_dtype, M, N, K, epilogue,
                                   preact_bf16, ld_preact, bias_grad, nullptr, dx, dx_dtype, ld_dx, accum, stream);
    } catch (...) {
        return fail(TE_ERR_INTERNAL, "te_fp8_gemm_dgrad_deterministic_noalloc: internal error");
    }
}

// The M-grouped data gradient; with `ws` set the per-expert bias gradient
// goes through that column-sum workspace and an ordered reduction instead of
// atomics.
static te_status_t mgrouped_dgrad(const char* fn, const void* dy, const float* dy_scales, te_dtype_t dy_dtype,
                                  const void* wt, const float* wt_scales, te_dtype_t wt_dtype, int64_t sum_m,
                                  int64_t N, int64_t K, int32_t G, const int32_t* m_block_group, uint32_t epilogue,
                                  const void* preact_bf16, int64_t ld_preact, float* bias_grad, float* ws, void* dx,
                                  te_dtype_t dx_dtype, int64_t ld_dx, te_accum_t accum, hipStream_t stream)
{
    if (!m_block_group) return fail(TE_ERR_INVALID_ARGUMENT, "%s: m_block_group is null", fn);
    if (!aligned(m_block_group, 4)) return fail(TE_ERR_MISALIGNED, "%s: m_block_group must be 4-byte aligned", fn);
    if (G < 1 || G > 1024) return fail(TE_ERR_INVALID_ARGUMENT, "%s: G must be in [1, 1024] (got %d)", fn, (int)G);
    if (sum_m < tefp8::kMGroupRows || sum_m % tefp8::kMGroupRows != 0)
        return fail(TE_ERR_INVALID_ARGUMENT, "%s: sum_m must be a positive multiple of %d (got %lld)", fn,
                    tefp8::kMGroupRows, (long long)sum_m);
    te_status_t st = check_operands(fn, dy, dy_scales, dy_dtype, wt, wt_scales, wt_dtype, sum_m, N, K, accum);
    if (st != TE_OK) return st;
    const uint32_t allowed = TE_EPI_DGELU | TE_EPI_BGRAD;
    if (epilogue & ~allowed) return fail(TE_ERR_INVALID_ARGUMENT, "%s: epilogue flags 0x%x are not dgrad flags", fn, epilogue);
    if (ws && !(epilogue & TE_EPI_BGRAD))
        return fail(TE_ERR_INVALID_ARGUMENT, "%s: the epilogue must include TE_EPI_BGRAD", fn);
    if (epilogue & TE_EPI_DGELU) {
        if (!preact_bf16) return fail(TE_ERR_INVALID_ARGUMENT, "%s: TE_EPI_DGELU needs preact_bf16", fn);
        if (ld_preact < N) return fail(TE_ERR_INVALID_ARGUMENT, "%s: ld_preact (%lld) is below N", fn, (long long)ld_preact);
        if (!aligned(preact_bf16, 16) || ld_preact % 8 != 0)
            return fail(TE_ERR_MISALIGNED, "%s: preact must be 16-byte aligned with ld_preact a multiple of 8", fn);
    } else if (preact_bf16) {
        return fail(TE_ERR_INVALID_ARGUMENT, "%s: preact given without TE_EPI_DGELU", fn);
    }
    if (epilogue & TE_EPI_BGRAD) {
        if (!bias_grad) return fail(TE_ERR_INVALID_ARGUMENT, "%s: TE_EPI_BGRAD needs bias_grad", fn);
        if (!aligned(bias_grad, 4)) return fail(TE_ERR_MISALIGNED, "%s: bias_grad must be 4-byte aligned", fn);
    } else if (bias_grad) {
        return fail(TE_ERR_INVALID_ARGUMENT, "%s: bias_grad given without TE_EPI_BGRAD", fn);
    }
    st = check_output(fn, "dx", dx, dx_dtype, ld_dx, N);
    if (st != TE_OK) return st;
    tefp8::GemmArgs g = base_args(dy, dy_scales, dy_dtype, wt, wt_scales, wt_dtype, sum_m, N, K, accum);
    g.epi = tefp8::Epi::Dgrad;
    g.flags = epilogue;
    g.out = dx;
    g.out_bf16 = dx_dtype == TE_DTYPE_BF16;
    g.ld_out = ld_dx;
    g.preact = static_cast<const uint16_t*>(preact_bf16);
    g.ld_aux = ld_preact;
    g.bias_grad = bias_grad;
    g.m_block_group = m_block_group;
    g.num_b_groups = G;
    g.b_group_stride = N * K;
    g.sb_group_stride = (K / 128) * te_scale_ld(N);
    g.bias_group_stride = N;
    if (ws) {
        g.bgrad_ws = ws;
        g.bgrad_ws_ld = (N + 3) / 4 * 4;
    } else if (epilogue & TE_EPI_BGRAD) {
        hipError_t e = tefp8::launch_zero_f32(bias_grad, (int64_t)G * N, stream);
        if (e != hipSuccess) return fail(TE_ERR_HIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
    }
    st = launch(fn, g, stream, K, dy_dtype, wt_dtype, accum, epilogue);
    if (st != TE_OK || !ws) return st;
    hipError_t e = tefp8::launch_mgrouped_bgrad_reduce(ws, sum_m / tefp8::kMGroupRows, g.bgrad_ws_ld, N, G,
                                                       m_block_group, bias_grad, stream);
    if (e != hipSuccess) return fail(TE_ERR_HIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

te_status_t te_fp8_mgrouped_gemm_dgrad(const void* dy, const float* dy_scales, te_dtype_t dy_dtype,
                                       const void* wt, const float* wt_scales, te_dtype_t wt_dtype,
                                       int64_t sum_m, int64_t N, int64_t K, int32_t G, const int32_t* m_block_group,
                                       uint32_t epilogue, const void* preact_bf16, int64_t ld_preact,
                                       float* bias_grad, void* dx, te_dtype_t dx_dtype, int64_t ld_dx,
                                       te_accum_t accum, hipStream_t stream)
{
    try {
        return mgrouped_dgrad("te_fp8_mgrouped_gemm_dgrad", dy, dy_scales, dy_dtype, wt, wt_scales, wt_dtype, sum_m,
                              N, K, G, m_block_group, epilogue, preact_bf16, ld_preact, bias_grad, nullptr, dx,
                              dx_dtype, ld_dx, accum, stream);
    } catch (...) {
        return fail(TE_ERR_INTERNAL, "te_fp8_mgrouped_gemm_dgrad: internal error");
    }
}

te_status_t te_fp8_mgrouped_gemm_dgrad_deterministic(const void* dy, const float* dy_scales, te_dtype_t dy_dtype,
                                                     const void* wt, const float* wt_scales, te_dtype_t wt_dtype,
                                                     int64_t sum_m, int64_t N, int64_t K, int32_t G,
                                                     const int32_t* m_block_group, uint32_t epilogue,
                                                     const void* preact_bf16, int64_t ld_preact, float* bias_grad,
                                                     void* workspace, int64_t workspace_bytes, void* dx,
                                                     te_dtype_t dx_dtype, int64_t ld_dx, te_accum_t accum,
                                                     hipStream_t stream)
{
    try {
        const char* fn = "te_fp8_mgrouped_gemm_dgrad_deterministic";
        if (!workspace) return fail(TE_ERR_INVALID_ARGUMENT, "%s: workspace is null", fn);
        if (!aligned(workspace, 16)) return fail(TE_ERR_MISALIGNED, "%s: workspace must be 16-byte aligned", fn);
        const int64_t need = te_fp8_dgrad_bgrad_workspace_bytes(sum_m, N);
        if (sum_m >= 1 && N >= 1 && workspace_bytes < need)
            return fail(TE_ERR_INVALID_ARGUMENT, "%s: workspace_bytes %lld below the %lld bytes needed", fn,
                        (long long)workspace_bytes, (long long)need);
        return mgrouped_dgrad(fn, dy, dy_scales, dy_dtype, wt, wt_scales, wt_dtype, sum_m, N, K, G, m_block_group,
                              epilogue, preact_bf16, ld_preact, bias_grad, static_cast<float*>(workspace), dx,
                              dx_dtype, ld_dx, accum, stream);
    } catch (...) {
        return fail(TE_ERR_INTERNAL, "te_fp8_mgrouped_gemm_dgrad_deterministic: internal error");
    }
}

}  // extern "C"
