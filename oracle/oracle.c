/*
 * CPU oracle for the scaled-FP8 Linear-layer GEMMs.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file; only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark use it.  It shares no code, header, table
 * or constant generator with the HIP library.
 *
 * Everything here is the plain definition of what the library computes,
 * evaluated in double precision on exactly the fp8 bytes and fp32 scales the
 * GPU consumes.  No blocking, fusion or reordering beyond the definitions is
 * done: one output element is one loop over K.  The only concession to speed
 * is an OpenMP parallel loop over independent outputs.
 *
 * Sources (the pages this implements):
 *  - "Replaced cublasLt calls with rocblas gemm + 6 manually crafted
 *    epilogues" (ROCm/TransformerEngine pull request 3), the maintainer's
 *    explanation of GEMM_m/GEMM_n: forward Y = X*W^T + b with X (m,k),
 *    W (n,k), Y (m,n) and b of length n; backward dX = dY*W, dW = dY^T*X,
 *    db = sum(dY, axis=0); the review note that the backward order matters
 *    when bias and GELU are both present; reductions kept in fp32.
 *  - "Weight gradient kernels for dense and MoE models" (DeepGEMM pull
 *    request 95): the wgrad kernel accumulates, out += x*y^T, not out = x*y^T;
 *    the grouped variant splits the contraction (K) dimension per expert;
 *    inputs are produced by a per-token cast to fp8.
 *  - "FP8 GEMM for the fprop should use fast accumulation" (openxla/xla
 *    issue 6168): e4m3 for the forward GEMM, e4m3 with e5m2 for the backward
 *    GEMMs; accumulation precision is a per-op choice.  Both policies must
 *    reach this same mathematical result, so the oracle has no policy input.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - fp8 formats are the OCP ones: E4M3FN (bias 7, no infinities, max 448,
 *    NaN = S.1111.111) and E5M2 (bias 15, IEEE-like, max 57344).
 *  - The per-token cast uses one fp32 scale per row and per 128 consecutive
 *    contraction elements.  s is the dequantisation multiplier (value = q*s):
 *        amax  = max |x| over the group,  amax_c = max(amax, 2^-100)
 *        s     = fl32(amax_c / FP8_MAX)
 *        q     = enc(fl32(x * fl32(FP8_MAX / amax_c)))
 *    and in power-of-two mode s = 2^j with j the smallest integer such that
 *    FP8_MAX * 2^j >= amax_c, q = enc(fl32(x * 2^-j)).
 *    enc() rounds to nearest, ties to even, and saturates to +-FP8_MAX.
 *  - GELU is the tanh form, 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).
 *  - In the backward pass dGELU is applied before the bias gradient.
 *
 *  - The library's other entry points reduce to these definitions, composed
 *    in the Python side of this package: the cast of X and of X^T (fused
 *    cast-transpose), the cast of an epilogue's fp32 result (quantising
 *    stores; oracle_cast_per_token_f32 below), and each 256-row block of an
 *    M-grouped GEMM through the dense forward or dgrad with its expert's
 *    operand.
 *
 * parity unpinned: the GELU form (the pages give none; the tanh form is fixed
 * here and pinned against a library implementation of that same form), and
 * the fast-accumulation policy's own precision (the pages state it is
 * undocumented; both policies are held to this single oracle).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_E4M3 1
#define ORACLE_E5M2 2

/* ------------------------------------------------------------------ codecs */

/* Exact value of one fp8 code, from the OCP bit-field definitions. */
double oracle_fp8_decode(uint8_t code, int fmt)
{
    int sign = code >> 7;
    double v;
    if (fmt == ORACLE_E4M3) {
        int e = (code >> 3) & 0xF, m = code & 0x7;
        if (e == 0xF && m == 0x7) return NAN;                 /* only NaN, no inf */
        if (e == 0) v = ldexp((double)m, -9);                 /* m/8 * 2^(1-7)    */
        else        v = ldexp(8.0 + m, e - 7 - 3);            /* (1+m/8) * 2^(e-7) */
    } else {
        int e = (code >> 2) & 0x1F, m = code & 0x3;
        if (e == 0x1F) return m ? NAN : (sign ? -INFINITY : INFINITY);
        if (e == 0) v = ldexp((double)m, -16);                /* m/4 * 2^(1-15)   */
        else        v = ldexp(4.0 + m, e - 15 - 2);           /* (1+m/4) * 2^(e-15) */
    }
    return sign ? -v : v;
}

static uint8_t max_code(int fmt) { return fmt == ORACLE_E4M3 ? 0x7E : 0x7B; }

double oracle_fp8_max(int fmt) { return oracle_fp8_decode(max_code(fmt), fmt); }

/*
 * Nearest finite code to v, ties to the even code (whose mantissa LSB is 0),
 * values beyond the largest finite magnitude saturate to it.  The positive
 * finite codes 0..max_code are increasing in value, so a bisection over them
 * finds the two neighbours of |v|.
 */
uint8_t oracle_fp8_encode(float v, int fmt)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    int hi = max_code(fmt);
    if (a >= oracle_fp8_decode((uint8_t)hi, fmt)) return (uint8_t)(sign | hi);
    int lo = 0;                                   /* dec(lo) <= a < dec(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (oracle_fp8_decode((uint8_t)mid, fmt) <= a) lo = mid; else hi = mid;
    }
    double dl = a - oracle_fp8_decode((uint8_t)lo, fmt);
    double dh = oracle_fp8_decode((uint8_t)hi, fmt) - a;
    int c = dl < dh ? lo : (dh < dl ? hi : ((lo & 1) ? hi : lo));
    return (uint8_t)(sign | c);
}

void oracle_fp8_decode_array(const uint8_t* q, int64_t n, int fmt, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp8_decode(q[i], fmt);
}

void oracle_fp8_encode_array(const float* v, int64_t n, int fmt, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp8_encode(v[i], fmt);
}

/* bf16 is the upper half of an fp32 bit pattern. */
float oracle_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* ------------------------------------------------------------------ cast */

/* Smallest j with fmax * 2^j >= a (a > 0, finite); every comparison is exact. */
static int pow2_exponent(float a, double fmax)
{
    int e;
    frexp((double)a / fmax, &e);                 /* estimate, then correct exactly */
    int j = e;
    while (ldexp(fmax, j - 1) >= (double)a) --j;
    while (ldexp(fmax, j) < (double)a) ++j;
    return j;
}

/*
 * One 128-element group of the per-token cast, from fp32 values: amax,
 * amax_c = max(amax, 2^-100), the dequantisation scale fl32(amax_c / FP8_MAX)
 * (or the power of two 2^j, j smallest with FP8_MAX 2^j >= amax_c) and the
 * codes enc(fl32(v * fl32(FP8_MAX / amax_c))) (or enc(v * 2^-j)).  Returns
 * the scale; *bad is set for a non-finite input.
 */
static float cast_group(const float* v, int fmt, int pow2, uint8_t* q, int* bad)
{
    const float fmax = (float)oracle_fp8_max(fmt);
    float amax = 0.0f;
    for (int i = 0; i < 128; ++i) {
        if (!isfinite(v[i])) *bad = 1;
        if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
    }
    float amax_c = amax > 0x1p-100f ? amax : 0x1p-100f;
    float scale, mult;
    if (pow2) {
        int j = pow2_exponent(amax_c, (double)fmax);
        scale = ldexpf(1.0f, j);
        mult = ldexpf(1.0f, -j);
    } else {
        scale = amax_c / fmax;
        mult = fmax / amax_c;
    }
    for (int i = 0; i < 128; ++i) {
        float prod = v[i] * mult;
        q[i] = oracle_fp8_encode(prod, fmt);
    }
    return scale;
}

/*
 * Per-token cast: x is bf16 [rows][cols] (row stride ld_x elements), cols a
 * multiple of 128.  Writes q [rows][cols] (row stride ld_q bytes) and
 * s [rows][cols/128].  Returns 0, or -1 for a non-finite input (undefined).
 */
int oracle_cast_per_token(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                          int fmt, int pow2, uint8_t* q, int64_t ld_q, float* s)
{
    const int64_t groups = cols / 128;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t g = 0; g < groups; ++g) {
            float v[128];
            for (int i = 0; i < 128; ++i) v[i] = oracle_bf16_to_f32(x[r * ld_x + g * 128 + i]);
            s[r * groups + g] = cast_group(v, fmt, pow2, q + r * ld_q + g * 128, &bad);
        }
    }
    return bad ? -1 : 0;
}

/*
 * The same cast of an fp32 matrix x [rows][cols] (row stride ld_x elements):
 * the per-token cast of a GEMM epilogue's fp32 result before any rounding.
 */
int oracle_cast_per_token_f32(const float* x, int64_t rows, int64_t cols, int64_t ld_x,
                              int fmt, int pow2, uint8_t* q, int64_t ld_q, float* s)
{
    const int64_t groups = cols / 128;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t g = 0; g < groups; ++g)
            s[r * groups + g] = cast_group(x + r * ld_x + g * 128, fmt, pow2, q + r * ld_q + g * 128, &bad);
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------ GEMM */

/*
 * One output of the block-scaled "NT" product: A is [M][K] and B is [N][K],
 * both contraction-contiguous (row strides lda, ldb bytes), scales
 * [M][K/128] and [N][K/128] (row strides lsa, lsb floats).
 *   o = sum_kb sA[m,kb] sB[n,kb] sum_{k in kb} dec(A[m,k]) dec(B[n,k])
 *   d = the same sum with every term replaced by its absolute value.
 * Columns k0 .. k0+K-1 are used (k0 a multiple of 128).
 */
static void dot_one(const uint8_t* qa, const float* sa, int fa, int64_t lda, int64_t lsa,
                    const uint8_t* qb, const float* sb, int fb, int64_t ldb, int64_t lsb,
                    int64_t m, int64_t n, int64_t k0, int64_t K,
                    const double* ta, const double* tb, double* o, double* d)
{
    (void)fa; (void)fb;
    double acc = 0.0, mag = 0.0;
    for (int64_t kb = k0 / 128; kb < (k0 + K) / 128; ++kb) {
        double blk = 0.0, blkmag = 0.0;
        for (int64_t k = kb * 128; k < kb * 128 + 128; ++k) {
            double p = ta[qa[m * lda + k]] * tb[qb[n * ldb + k]];
            blk += p;
            blkmag += fabs(p);
        }
        double sc = (double)sa[m * lsa + kb] * (double)sb[n * lsb + kb];
        acc += sc * blk;
        mag += fabs(sc) * blkmag;
    }
    *o = acc;
    *d = mag;
}

static void decode_table(int fmt, double t[256])
{
    for (int c = 0; c < 256; ++c) t[c] = oracle_fp8_decode((uint8_t)c, fmt);
}

/* Full product o[M][N], d[M][N] over contraction columns [k0, k0+K). */
void oracle_gemm_nt(const uint8_t* qa, const float* sa, int fa, int64_t lda, int64_t lsa,
                    const uint8_t* qb, const float* sb, int fb, int64_t ldb, int64_t lsb,
                    int64_t M, int64_t N, int64_t k0, int64_t K, double* o, double* d)
{
    double ta[256], tb[256];
    decode_table(fa, ta);
    decode_table(fb, tb);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            dot_one(qa, sa, fa, lda, lsa, qb, sb, fb, ldb, lsb, m, n, k0, K, ta, tb,
                    &o[m * N + n], &d[m * N + n]);
}

/* The same product at a list of (m, n) positions only. */
void oracle_gemm_nt_entries(const uint8_t* qa, const float* sa, int fa, int64_t lda, int64_t lsa,
                            const uint8_t* qb, const float* sb, int fb, int64_t ldb, int64_t lsb,
                            int64_t k0, int64_t K, const int64_t* mi, const int64_t* ni,
                            int64_t count, double* o, double* d)
{
    double ta[256], tb[256];
    decode_table(fa, ta);
    decode_table(fb, tb);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i)
        dot_one(qa, sa, fa, lda, lsa, qb, sb, fb, ldb, lsb, mi[i], ni[i], k0, K, ta, tb,
                &o[i], &d[i]);
}

/* ------------------------------------------------------------- epilogues */

static const double GELU_C = 0.79788456080286535588;   /* sqrt(2/pi) */
static const double GELU_A = 0.044715;

double oracle_gelu(double z)
{
    return 0.5 * z * (1.0 + tanh(GELU_C * (z + GELU_A * z * z * z)));
}

/* d/dz of oracle_gelu. */
double oracle_dgelu(double z)
{
    double t = tanh(GELU_C * (z + GELU_A * z * z * z));
    return 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * GELU_C * (1.0 + 3.0 * GELU_A * z * z);
}

/*
 * Forward epilogue on a product o/d of shape [M][N]:
 *   z = o + b[n]  (b bf16, optional);  y = GELU(z) if gelu else z.
 * zmag = d + |b[n]| is the magnitude scale of z.
 */
void oracle_fwd_epilogue(const double* o, const double* d, int64_t M, int64_t N,
                         const uint16_t* bias, int gelu, double* z, double* zmag, double* y)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double b = bias ? (double)oracle_bf16_to_f32(bias[n]) : 0.0;
            double zz = o[m * N + n] + b;
            z[m * N + n] = zz;
            zmag[m * N + n] = d[m * N + n] + fabs(b);
            y[m * N + n] = gelu ? oracle_gelu(zz) : zz;
        }
}

/*
 * Backward epilogue: D = o, times GELU'(z) at the saved bf16 pre-activation
 * when preact is given; then db[n] = sum over the M rows of D (after the
 * dGELU).  Dmag and dbmag carry the magnitude scales d*|GELU'| and its sum.
 */
void oracle_dgrad_epilogue(const double* o, const double* d, int64_t M, int64_t N,
                           const uint16_t* preact, int64_t ld_preact,
                           double* D, double* Dmag, double* db, double* dbmag)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double g = preact ? oracle_dgelu((double)oracle_bf16_to_f32(preact[m * ld_preact + n])) : 1.0;
            D[m * N + n] = o[m * N + n] * g;
            Dmag[m * N + n] = d[m * N + n] * fabs(g);
        }
    if (db) {
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0, sm = 0.0;
            for (int64_t m = 0; m < M; ++m) { s += D[m * N + n]; sm += Dmag[m * N + n]; }
            db[n] = s;
            dbmag[n] = sm;
        }
    }
}

/* wgrad: out' = out + o (out as it was before the call); mag = |out| + d. */
void oracle_wgrad(const double* o, const double* d, const float* out_init, int64_t M, int64_t N,
                  int64_t ld_out, double* out_new, double* mag)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double init = (double)out_init[m * ld_out + n];
            out_new[m * N + n] = init + o[m * N + n];
            mag[m * N + n] = fabs(init) + d[m * N + n];
        }
}

/*
 * K-grouped wgrad: A is [M][sumK], B is [N][sumK]; group g owns contraction
 * columns [off_g, off_g + K_g) with off_g = K_0 + ... + K_(g-1), and
 *   out[g] += A[:, group g] * B[:, group g]^T.
 * A group with K_g = 0 leaves out[g] as it was.  out_init/out_new/mag are
 * [G][M][N] contiguous.
 */
void oracle_kgrouped_wgrad(const uint8_t* qa, const float* sa, int fa,
                           const uint8_t* qb, const float* sb, int fb,
                           int64_t M, int64_t N, const int64_t* group_k, int G,
                           const float* out_init, double* out_new, double* mag)
{
    int64_t sumk = 0;
    for (int g = 0; g < G; ++g) sumk += group_k[g];
    double ta[256], tb[256];
    decode_table(fa, ta);
    decode_table(fb, tb);
    int64_t off = 0;
    for (int g = 0; g < G; ++g) {
        const float* oi = out_init + (int64_t)g * M * N;
        double* on = out_new + (int64_t)g * M * N;
        double* mg = mag + (int64_t)g * M * N;
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t m = 0; m < M; ++m)
            for (int64_t n = 0; n < N; ++n) {
                double o = 0.0, d = 0.0;
                if (group_k[g] > 0)
                    dot_one(qa, sa, fa, sumk, sumk / 128, qb, sb, fb, sumk, sumk / 128,
                            m, n, off, group_k[g], ta, tb, &o, &d);
                on[m * N + n] = (double)oi[m * N + n] + o;
                mg[m * N + n] = fabs((double)oi[m * N + n]) + d;
            }
        off += group_k[g];
    }
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
