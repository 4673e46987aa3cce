// Block-scaled FP8 "NT" GEMM for gfx950 with fused Linear-layer epilogues.
//
//   D[m][n] = sum_kb sA[m][kb] sB[n][kb] sum_{k in kb} qA[m][k] qB[n][k]
//
// A [M][K] and B [N][K] are fp8 (E4M3 or E5M2), contraction-contiguous, with
// one fp32 scale per row per 128-deep block.  Which products of a Linear layer
// map onto this form, and the epilogues, follow the maintainer's explanation
// on "Replaced cublasLt calls with rocblas gemm + 6 manually crafted
// epilogues" (forward Y = X W^T + b with b of length n; dX = dY W; dW = dY^T
// X; db = column sum of the gradient; dGELU before the bias gradient), and
// the weight-gradient "out +=" semantics and K-grouped form of "Weight
// gradient kernels for dense and MoE models".
//
// Design for CDNA4 (gfx950):
//  * Workgroup tile 256 x 256, eight waves (2 along M x 4 along N), each wave
//    owning 128 x 64 outputs = 8 x 4 matrix-core tiles of 16 x 16.  Eight
//    waves give two waves per SIMD so that one wave's matrix-core work can
//    overlap the other's vector work (the FULL promotion and the epilogue).
//  * One 128-deep contraction block is one v_mfma_f32_16x16x128_f8f6f4, which
//    is exactly one scale block: FULL starts it from zero and promotes
//    acc += P * (sA * sB) in fp32 FMA; FAST passes the two E8M0 exponents of
//    power-of-two scales to v_mfma_scale_f32_16x16x128_f8f6f4 and chains the
//    accumulator through the matrix core (no vector work), falling back to
//    the FULL update for any block whose scales are not powers of two.
//  * The B tile is the instruction's first operand, so each lane's four
//    accumulator registers are four consecutive n of one row m: stores are
//    16-byte (fp32) / 8-byte (bf16) vectors along the output row.
//  * Operands stream global -> LDS with global_load_lds_dwordx4 (no register
//    staging), double-buffered: while the matrix cores consume stage s, the
//    loads for stage s+1 are in flight (restrict-qualified stage pointers keep
//    the compiler from making this stage's reads wait for them, and the
//    barrier carries no fence that would drain them).  Each 128-byte LDS row stores its
//    16-byte chunk c at slot c ^ ((row >> 1) & 7), so the 16 rows read by one
//    16-lane group of a ds_read_b128 fall in 16 distinct 16-byte bank groups.
//    The two scale vectors of the block ride along in the same stage.
//  * Edge tiles clamp their load rows to the last valid row (no faults, the
//    values are unused) and mask their stores.
//  * K-grouped launches carry up to 128 (kb_off, kb_len, out) descriptors by
//    value; blocks are ordered longest group first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "te_fp8.h"

namespace tefp8 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kBM = 256, kBN = 256, kBK = 128;
constexpr int kWavesM = 2, kWavesN = 4;
constexpr int kThreads = 64 * kWavesM * kWavesN;  // 512
constexpr int kWM = kBM / kWavesM;                // 128
constexpr int kWN = kBN / kWavesN;                // 64
constexpr int kTM = kWM / 16;                     // 8
constexpr int kTN = kWN / 16;                     // 4
constexpr int kTileA = kBM * kBK;                 // 32 KiB
constexpr int kTileB = kBN * kBK;                 // 32 KiB
constexpr int kStageBytes = kTileA + kTileB + (kBM + kBN) * 4;
constexpr int kStages = 2;
constexpr int kGroupM = 8;                        // tile rows per raster group

static_assert(kBM * kBK / 16 == kThreads * 4, "A tile = four 16-byte loads per thread");
static_assert(kBN * kBK / 16 == kThreads * 4, "B tile = four 16-byte loads per thread");
static_assert(kBM + kBN == kThreads, "one scale per thread per stage");

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ ((row >> 1) & 7)) << 4); }

// Per-tile buffer resources: bases at the tile's first row, ranges cut at the
// last valid row (rows past it read as zero: no clamping, no faults).
struct TileSrc {
    __amdgpu_buffer_rsrc_t a, b, sa, sb;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)min(bytes, (int64_t)0x7FFFFFFF),
                                             0x00020000);
}

__device__ __forceinline__ TileSrc tile_src(const GemmArgs& p, int64_t m0, int64_t n0)
{
    TileSrc s;
    s.a = make_rsrc(p.a + m0 * p.lda, min((int64_t)kBM, p.M - m0) * p.lda);
    s.b = make_rsrc(p.b + n0 * p.ldb, min((int64_t)kBN, p.N - n0) * p.ldb);
    s.sa = make_rsrc(p.sa + m0 * p.lsa, min((int64_t)kBM, p.M - m0) * p.lsa * 4);
    s.sb = make_rsrc(p.sb + n0 * p.lsb, min((int64_t)kBN, p.N - n0) * p.lsb * 4);
    return s;
}

// Issue the global -> LDS copies of one 128-deep stage (A tile, B tile, scales).
__device__ __forceinline__ void load_stage(const GemmArgs& p, const TileSrc& src, uint8_t* stage, int kb, int wave,
                                           int lane)
{
    const int kcol = kb * kBK;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int blk = wave * 4 + t;                 // 1 KiB block = 8 rows of 128 bytes
        const int ci = blk * 64 + lane;               // 16-byte chunk index within the tile
        const int row = ci >> 3;
        const int chunk = (ci & 7) ^ ((row >> 1) & 7);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src.a, (lds_ptr_t)(stage + blk * 1024), 16,
                                                 (uint32_t)(row * p.lda + chunk * 16), kcol, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src.b, (lds_ptr_t)(stage + kTileA + blk * 1024), 16,
                                                 (uint32_t)(row * p.ldb + chunk * 16), kcol, 0, 0);
    }
    // scales: waves 0-3 fetch sA for the 256 tile rows, waves 4-7 sB for the 256 tile columns
    const bool is_a = wave < 4;
    const int r = (is_a ? wave : wave - 4) * 64 + lane;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? src.sa : src.sb, (lds_ptr_t)(stage + kTileA + kTileB + wave * 256),
                                             4, (uint32_t)(r * (is_a ? p.lsa : p.lsb) * 4), kb * 4, 0, 0);
}

__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int row, int q4)
{
    const uint4 lo = *reinterpret_cast<const uint4*>(tile + swz(row, q4));
    const uint4 hi = *reinterpret_cast<const uint4*>(tile + swz(row, q4 + 4));
    v8i f;
    f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
    f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
    return f;
}

__device__ __forceinline__ bool is_pow2_scale(float s)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, s);
    const uint32_t e = u >> 23;
    return (u & 0x007FFFFFu) == 0 && e != 0 && e < 255;  // positive normal power of two
}

__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __builtin_bit_cast(float, h << 16); }

// GELU, tanh form: 0.5 z (1 + tanh(u)) = z / (1 + exp(-2u)), u = sqrt(2/pi)(z + 0.044715 z^3).
constexpr float kGeluC = 0.7978845608028654f;
constexpr float kGeluA = 0.044715f;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float gelu_exp2_arg(float z)
{
    // -2u * log2(e), so exp(-2u) = exp2(result)
    return z * fmaf(z * z, -2.0f * kGeluC * kGeluA * kLog2e, -2.0f * kGeluC * kLog2e);
}

__device__ __forceinline__ float gelu(float z)
{
    const float e = __builtin_amdgcn_exp2f(gelu_exp2_arg(z));
    return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// d/dz of the tanh-form GELU: sigma + 2 z sigma (1 - sigma) sqrt(2/pi) (1 + 3 a z^2), sigma = 1/(1+exp(-2u)).
__device__ __forceinline__ float dgelu(float z)
{
    const float e = __builtin_amdgcn_exp2f(fminf(gelu_exp2_arg(z), 64.0f));
    const float s = __builtin_amdgcn_rcpf(1.0f + e);
    const float one_minus_s = e * s;
    const float z2 = z * z;
    return fmaf(2.0f * kGeluC * z * s * one_minus_s, fmaf(3.0f * kGeluA, z2, 1.0f), s);
}

// Workgroup barrier without a memory fence: callers wait for their own
// global->LDS copies explicitly; this waits for the wave's own LDS reads and
// syncs.  (A fenced __syncthreads() would also drain the next stage's copies.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One contraction block, held in `stage`; the copies of the next block go to
// `other`.  The two stages are restrict-qualified so the compiler knows the
// copies into `other` do not feed the reads of `stage` and does not make
// those reads wait for them: the next block's copies overlap this block's
// matrix-core work.  kChain: every scale is a power of two and the block
// scales ride in the matrix-core instruction; otherwise each block's product
// starts from zero and is promoted in fp32.
template <int kFmtA, int kFmtB, bool kChain>
__device__ __forceinline__ void block_step(const GemmArgs& p, uint8_t* __restrict__ stage,
                                           uint8_t* __restrict__ other, v4f (&acc)[kTM][kTN], const TileSrc& src,
                                           int kb0, int it, int nkb, int wave, int lane)
{
    const int wm = wave / kWavesN, wn = wave % kWavesN;
    const int r16 = lane & 15, q4 = lane >> 4;
    // this block's copies (the only ones in flight) have landed everywhere, and
    // every wave is done reading `other` (the previous block)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (it + 1 < nkb) load_stage(p, src, other, kb0 + it + 1, wave, lane);

    const uint8_t* As = stage;
    const uint8_t* Bs = stage + kTileA;
    const float* sAs = reinterpret_cast<const float*>(stage + kTileA + kTileB);
    const float* sBs = sAs + kBM;

    v8i bf[kTN];
#pragma unroll
    for (int j = 0; j < kTN; ++j) bf[j] = read_frag(Bs, wn * kWN + j * 16 + r16, q4);

    if (kChain) {
        // E8M0 exponent of a positive normal power of two = its fp32 exponent field
        int eb[kTN];
#pragma unroll
        for (int j = 0; j < kTN; ++j) eb[j] = (int)(__builtin_bit_cast(uint32_t, sBs[wn * kWN + j * 16 + r16]) >> 23);
        v8i afq[3];
        int eaq[3];
#pragma unroll
        for (int d = 0; d < 3 - 1; ++d) {
            afq[d] = read_frag(As, wm * kWM + d * 16 + r16, q4);
            eaq[d] = (int)(__builtin_bit_cast(uint32_t, sAs[wm * kWM + d * 16 + r16]) >> 23);
        }
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
            if (i + 3 - 1 < kTM) {
                afq[(i + 3 - 1) % 3] = read_frag(As, wm * kWM + (i + 3 - 1) * 16 + r16, q4);
                eaq[(i + 3 - 1) % 3] = (int)(__builtin_bit_cast(uint32_t, sAs[wm * kWM + (i + 3 - 1) * 16 + r16]) >> 23);
            }
            const v8i af = afq[i % 3];
            const int ea = eaq[i % 3];
#pragma unroll
            for (int j = 0; j < kTN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, acc[i][j], kFmtB, kFmtA, 0,
                                                                             eb[j], 0, ea);
        }
    } else {
        float4 sb[kTN];
#pragma unroll
        for (int j = 0; j < kTN; ++j) sb[j] = *reinterpret_cast<const float4*>(sBs + wn * kWN + j * 16 + q4 * 4);
        v8i afq[3];
        float saq[3];
#pragma unroll
        for (int d = 0; d < 3 - 1; ++d) {
            afq[d] = read_frag(As, wm * kWM + d * 16 + r16, q4);
            saq[d] = sAs[wm * kWM + d * 16 + r16];
        }
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
            if (i + 3 - 1 < kTM) {
                afq[(i + 3 - 1) % 3] = read_frag(As, wm * kWM + (i + 3 - 1) * 16 + r16, q4);
                saq[(i + 3 - 1) % 3] = sAs[wm * kWM + (i + 3 - 1) * 16 + r16];
            }
            const v8i af = afq[i % 3];
            const float sa = saq[i % 3];
#pragma unroll
            for (int j = 0; j < kTN; ++j) {
                const v4f P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, v4f{0.f, 0.f, 0.f, 0.f},
                                                                               kFmtB, kFmtA, 0, 0, 0, 0);
                acc[i][j][0] = fmaf(P[0], sa * sb[j].x, acc[i][j][0]);
                acc[i][j][1] = fmaf(P[1], sa * sb[j].y, acc[i][j][1]);
                acc[i][j][2] = fmaf(P[2], sa * sb[j].z, acc[i][j][2]);
                acc[i][j][3] = fmaf(P[3], sa * sb[j].w, acc[i][j][3]);
            }
        }
    }
}

// The contraction loop over a double-buffered pair of stages; stage 0 has
// been issued by the caller.
template <int kFmtA, int kFmtB, bool kChain>
__device__ __forceinline__ void main_loop(const GemmArgs& p, uint8_t* smem, v4f (&acc)[kTM][kTN],
                                          const TileSrc& src, int kb0, int nkb, int wave, int lane)
{
    for (int it = 0; it < nkb; ++it) {
        uint8_t* cur = smem + (it & 1) * kStageBytes;
        uint8_t* oth = smem + ((it + 1) & 1) * kStageBytes;
        block_step<kFmtA, kFmtB, kChain>(p, cur, oth, acc, src, kb0, it, nkb, wave, lane);
    }
}

template <int kFmtA, int kFmtB, bool kFast, int kEpi>
__global__ __launch_bounds__(kThreads) void gemm_nt_kernel(const GemmArgs p)
{
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / kWavesN, wn = wave % kWavesN;
    const int r16 = lane & 15, q4 = lane >> 4;

    // ---- which group and tile this workgroup owns
    const int64_t tiles_m = (p.M + kBM - 1) / kBM;
    const int64_t tiles_n = (p.N + kBN - 1) / kBN;
    const int64_t tiles_per_group = tiles_m * tiles_n;
    const int gslot = (int)(blockIdx.x / tiles_per_group);
    int64_t t = blockIdx.x - (int64_t)gslot * tiles_per_group;
    const int64_t per_band = (int64_t)kGroupM * tiles_n;
    const int64_t band = t / per_band;
    const int64_t first_m = band * kGroupM;
    const int64_t band_rows = min((int64_t)kGroupM, tiles_m - first_m);
    t -= band * per_band;
    const int64_t m0 = (first_m + t % band_rows) * kBM;
    const int64_t n0 = (t / band_rows) * kBN;

    const Group grp = p.groups[gslot];
    const int kb0 = grp.kb_off, nkb = grp.kb_len;

    v4f acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const TileSrc src = tile_src(p, m0, n0);
    load_stage(p, src, smem, kb0, wave, lane);

    if (kFast) {
        // The scaled matrix-core chain is exact only for power-of-two scales:
        // take it when every scale of this tile's rows and columns over the
        // contraction range is one, otherwise promote like FULL.
        const int tid = threadIdx.x;
        const float* srow = tid < kBM ? p.sa + min(m0 + tid, p.M - 1) * p.lsa
                                      : p.sb + min(n0 + (tid - kBM), p.N - 1) * p.lsb;
        // independent loads (no short-circuit), so they are all in flight at once
        bool ok = true;
        for (int kb = kb0; kb < kb0 + nkb; ++kb) ok &= is_pow2_scale(srow[kb]);
        if (__syncthreads_and(ok)) {
            main_loop<kFmtA, kFmtB, true>(p, smem, acc, src, kb0, nkb, wave, lane);
        } else {
            main_loop<kFmtA, kFmtB, false>(p, smem, acc, src, kb0, nkb, wave, lane);
        }
    } else {
        main_loop<kFmtA, kFmtB, false>(p, smem, acc, src, kb0, nkb, wave, lane);
    }

    // ---- epilogue: lane holds D[m][n..n+3] for every (i, j)
    const int64_t out_off = (int64_t)grp.out_idx * p.out_group_stride;
    float colsum[kTN][4];
    if (kEpi == (int)Epi::Dgrad) {
#pragma unroll
        for (int j = 0; j < kTN; ++j) colsum[j][0] = colsum[j][1] = colsum[j][2] = colsum[j][3] = 0.f;
    }
    const bool has_bias = (p.flags & TE_EPI_BIAS) != 0;
    const bool has_gelu = (p.flags & TE_EPI_GELU) != 0;
    const bool has_aux = (p.flags & TE_EPI_AUX_PREACT) != 0;
    const bool has_dgelu = (p.flags & TE_EPI_DGELU) != 0;
    const bool has_bgrad = (p.flags & TE_EPI_BGRAD) != 0;

#pragma unroll
    for (int j = 0; j < kTN; ++j) {
        const int64_t n = n0 + wn * kWN + j * 16 + q4 * 4;
        const bool full4 = n + 3 < p.N;
        float bias[4] = {0.f, 0.f, 0.f, 0.f};
        if (kEpi == (int)Epi::Fwd && has_bias) {
            if (full4) {
                const uint2 bv = *reinterpret_cast<const uint2*>(p.bias + n);
                bias[0] = bf16_to_f32(bv.x & 0xFFFF); bias[1] = bf16_to_f32(bv.x >> 16);
                bias[2] = bf16_to_f32(bv.y & 0xFFFF); bias[3] = bf16_to_f32(bv.y >> 16);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) if (n + r < p.N) bias[r] = bf16_to_f32(p.bias[n + r]);
            }
        }
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
            const int64_t m = m0 + wm * kWM + i * 16 + r16;
            if (m >= p.M || n >= p.N) continue;
            float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
            if (kEpi == (int)Epi::Wgrad) {
                float* o = reinterpret_cast<float*>(p.out) + out_off + m * p.ld_out + n;
                if (full4) {
                    float4 cur = *reinterpret_cast<float4*>(o);
                    cur.x += v[0]; cur.y += v[1]; cur.z += v[2]; cur.w += v[3];
                    *reinterpret_cast<float4*>(o) = cur;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) if (n + r < p.N) o[r] += v[r];
                }
                continue;
            }
            if (kEpi == (int)Epi::Fwd) {
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] += bias[r];
                if (has_aux) {
                    uint16_t* a = p.aux + m * p.ld_aux + n;
                    if (full4) {
                        *reinterpret_cast<uint2*>(a) = make_uint2(bf16_rne(v[0]) | (bf16_rne(v[1]) << 16),
                                                                  bf16_rne(v[2]) | (bf16_rne(v[3]) << 16));
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) if (n + r < p.N) a[r] = (uint16_t)bf16_rne(v[r]);
                    }
                }
                if (has_gelu) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = gelu(v[r]);
                }
            } else {  // Dgrad
                if (has_dgelu) {
                    const uint16_t* z = p.preact + m * p.ld_aux + n;
                    float zf[4];
                    if (full4) {
                        const uint2 zv = *reinterpret_cast<const uint2*>(z);
                        zf[0] = bf16_to_f32(zv.x & 0xFFFF); zf[1] = bf16_to_f32(zv.x >> 16);
                        zf[2] = bf16_to_f32(zv.y & 0xFFFF); zf[3] = bf16_to_f32(zv.y >> 16);
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) zf[r] = n + r < p.N ? bf16_to_f32(z[r]) : 0.f;
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] *= dgelu(zf[r]);
                }
                if (has_bgrad) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) colsum[j][r] += v[r];
                }
            }
            // store y / dx
            if (p.out_bf16) {
                uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + out_off + m * p.ld_out + n;
                if (full4) {
                    *reinterpret_cast<uint2*>(o) = make_uint2(bf16_rne(v[0]) | (bf16_rne(v[1]) << 16),
                                                              bf16_rne(v[2]) | (bf16_rne(v[3]) << 16));
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) if (n + r < p.N) o[r] = (uint16_t)bf16_rne(v[r]);
                }
            } else {
                float* o = reinterpret_cast<float*>(p.out) + out_off + m * p.ld_out + n;
                if (full4) {
                    *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) if (n + r < p.N) o[r] = v[r];
                }
            }
        }
    }

    if (kEpi == (int)Epi::Dgrad && has_bgrad) {
        // column sums: reduce over the 16 lanes that share q4 (different m), one atomic per column
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float s = colsum[j][r];
                s += __shfl_xor(s, 1);
                s += __shfl_xor(s, 2);
                s += __shfl_xor(s, 4);
                s += __shfl_xor(s, 8);
                colsum[j][r] = s;
            }
            const int64_t n = n0 + wn * kWN + j * 16 + q4 * 4;
            if (r16 == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < p.N) unsafeAtomicAdd(p.bias_grad + n + r, colsum[j][r]);
            }
        }
    }
}

__global__ void zero_f32_kernel(float* p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

template <int kFmtA, int kFmtB, bool kFast>
hipError_t launch_epi(const GemmArgs& a, dim3 grid, hipStream_t s)
{
    switch (a.epi) {
    case Epi::Wgrad: gemm_nt_kernel<kFmtA, kFmtB, kFast, (int)Epi::Wgrad><<<grid, kThreads, 0, s>>>(a); break;
    case Epi::Fwd: gemm_nt_kernel<kFmtA, kFmtB, kFast, (int)Epi::Fwd><<<grid, kThreads, 0, s>>>(a); break;
    case Epi::Dgrad: gemm_nt_kernel<kFmtA, kFmtB, kFast, (int)Epi::Dgrad><<<grid, kThreads, 0, s>>>(a); break;
    }
    return hipGetLastError();
}

template <int kFmtA, int kFmtB>
hipError_t launch_policy(const GemmArgs& a, dim3 grid, hipStream_t s)
{
    return a.fast ? launch_epi<kFmtA, kFmtB, true>(a, grid, s) : launch_epi<kFmtA, kFmtB, false>(a, grid, s);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream, LaunchInfo* info)
{
    const int64_t tiles = ((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN);
    const int64_t blocks = tiles * a.num_groups;
    if (info) { info->tile_m = kBM; info->tile_n = kBN; info->threads = kThreads; info->grid = blocks; }
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks);
    if (a.fmt_a == FMT_E4M3 && a.fmt_b == FMT_E4M3) return launch_policy<FMT_E4M3, FMT_E4M3>(a, grid, stream);
    if (a.fmt_a == FMT_E5M2 && a.fmt_b == FMT_E4M3) return launch_policy<FMT_E5M2, FMT_E4M3>(a, grid, stream);
    if (a.fmt_a == FMT_E4M3 && a.fmt_b == FMT_E5M2) return launch_policy<FMT_E4M3, FMT_E5M2>(a, grid, stream);
    return launch_policy<FMT_E5M2, FMT_E5M2>(a, grid, stream);
}

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    zero_f32_kernel<<<(unsigned)blocks, 256, 0, stream>>>(p, n);
    return hipGetLastError();
}

}  // namespace tefp8
