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
//  * Workgroup tile 256 x 256, eight waves (4 along M x 2 along N), each wave
//    owning 64 x 128 outputs = 4 x 8 matrix-core tiles of 16 x 16 in VGPRs.
//    Two waves per SIMD: one wave's matrix-core work overlaps the other's
//    vector work (the FULL promotion, the epilogue) and LDS waits.
//  * One 128-deep contraction block is one v_mfma_f32_16x16x128_f8f6f4, which
//    is exactly one scale block.  FULL starts each block's product from zero
//    and promotes acc += P * (sA * sB) in fp32 FMA.  FAST, on a tile whose
//    scales over the whole contraction are powers of two, passes their E8M0
//    exponents to v_mfma_scale_f32_16x16x128_f8f6f4 and chains the
//    accumulator through the matrix core with no vector work; any other tile
//    is promoted like FULL.
//  * The B tile is the instruction's first operand, so each lane's four
//    accumulator registers are four consecutive n of one row m.  The wgrad
//    update reads and writes them as one 16-byte vector; the Linear-layer
//    epilogues first pair neighbouring column groups across lanes so that
//    every lane owns eight consecutive columns (16-byte bf16 runs).
//  * Operands stream global -> LDS with buffer_load ... lds (no register
//    staging) into two stages.  Each 128-byte LDS row stores its 16-byte chunk
//    c at slot c ^ ((row >> 1) & 7), so the 16 rows read by one 16-lane group
//    of a ds_read_b128 fall in 16 distinct bank groups.  The two scale vectors
//    of the block ride along in the same stage.
//  * Software pipeline inside a block: a wave keeps its four A fragments in
//    registers and streams its eight B column groups two groups ahead; in the
//    FULL loop each matrix-core product is promoted two instructions later
//    (the promotion of product t-2 precedes instruction t, which reuses its
//    register), so the vector unit never waits for the product just issued.
//    The single barrier of a block sits after the last read of the current
//    stage: past it the copies of block +2 go into the current stage and the
//    next block's first fragments are read from the other one, so a block
//    starts with its operands already in registers.  Slots are fenced with
//    scheduling barriers so the compiler keeps this order.
//  * Tiles past the last row read zero (buffer ranges end at the last valid
//    row) and their stores are masked.
//  * K-grouped launches carry up to 128 (kb_off, kb_len, out) descriptors by
//    value; blocks are ordered longest group first.  With group sizes in
//    device memory each tile derives its group's range from them instead
//    (every group has the same M x N tiles, so the tile -> group mapping needs
//    no sizes); a tile of an empty group does nothing.
//  * M-grouped launches (mixture-of-experts forward / data gradient) read the
//    expert of each 256-row block of A from device memory and take that
//    expert's B, B scales and bias; a block marked -1 is skipped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <cstdlib>
#include <cstring>

#ifndef TE_GEMM_PART
#define TE_GEMM_PART -1
#endif

#include "fp8_codec.h"
#include "internal.h"
#include "te_fp8.h"

namespace tefp8 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kBM = 256, kBN = 256, kBK = 128;
constexpr int kTileA = kBM * kBK;                 // 32 KiB
constexpr int kTileB = kBN * kBK;                 // 32 KiB
constexpr int kScaleBytes = (kBM + kBN) * 4;
constexpr int kSinkBytes = 1024;                  // target of the scale copies of waves that have none
constexpr int kStageBytes = kTileA + kTileB + kScaleBytes + kSinkBytes;
constexpr int kGroupM = 8;                        // tile rows per raster group
constexpr int kXcds = 8;                          // accelerator complex dies (each with its own L2)

constexpr int kWavesM = 4, kWavesN = 2;
constexpr int kWaves = kWavesM * kWavesN;
constexpr int kThreads = 64 * kWaves;             // 512
constexpr int kWM = kBM / kWavesM;                // 64 rows per wave
constexpr int kWN = kBN / kWavesN;                // 128 columns per wave
constexpr int kTM = kWM / 16;                     // 4 A fragments
constexpr int kTN = kWN / 16;                     // 8 B column groups
constexpr int kOpPerWave = (kBM / 8) / kWaves;    // 1 KiB copies of A (and of B) per wave
constexpr int kBarrierGroup = kTN - 2;            // the block's barrier precedes this column group
static_assert(kTM == 4 && kTN == 8 && kWaves * 64 == kBM + kBN, "layout assumed below");
static_assert(kMGroupRows == kBM, "an M-grouped block is one tile row");
static_assert(kBgradRowsPerTile == kWavesM, "one bias-gradient workspace row per wave along M");

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ ((row >> 1) & 7)) << 4); }

// Per-tile buffer resources: bases at the tile's first row, ranges cut at the
// last valid row (rows past it read as zero: no clamping, no faults).
struct TileSrc {
    __amdgpu_buffer_rsrc_t a, b;
    const float* sa;   // the tile's first row in block 0 of the block-major scales
    const float* sb;
    int sa_bytes, sb_bytes;  // valid scale bytes of one block (rows past the scale array's width read zero)
};

// The scale run this wave copies per block: wave 0 the tile rows' (A), wave 1
// the tile columns' (B), the others nothing (an empty range into the sink).
// The stride between blocks is made opaque once per tile so that it stays in
// a register: otherwise the compiler reloads it from the kernel arguments
// inside the loop and the wait for that load also drains the LDS reads.
struct ScaleSrc {
    const float* base;
    int64_t ld;        // floats between consecutive blocks
    int bytes;
    int dst;           // LDS offset of the run inside a stage
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)min(bytes, (int64_t)0x7FFFFFFF),
                                             0x00020000);
}

__device__ __forceinline__ TileSrc tile_src(const GemmArgs& p, int64_t m0, int64_t n0, int64_t bgrp)
{
    TileSrc s;
    s.a = make_rsrc(p.a + m0 * p.lda, min((int64_t)kBM, p.M - m0) * p.lda);
    s.b = make_rsrc(p.b + bgrp * p.b_group_stride + n0 * p.ldb, min((int64_t)kBN, p.N - n0) * p.ldb);
    s.sa = p.sa + m0;
    s.sb = p.sb + bgrp * p.sb_group_stride + n0;
    s.sa_bytes = (int)(min((int64_t)kBM, p.lsa - m0) * 4);
    s.sb_bytes = (int)(min((int64_t)kBN, p.lsb - n0) * 4);
    return s;
}

// The same tile with empty ranges: every copy reads zero and touches no
// memory.  Used for the copies past the last block so that the loop body is
// one straight-line block (no branch for the scheduler to sink work across).
__device__ __forceinline__ TileSrc select_src(const TileSrc& s, bool live)
{
    TileSrc e = s;
    e.a = live ? s.a : __builtin_amdgcn_make_buffer_rsrc(nullptr, 0, 0, 0x00020000);
    e.b = live ? s.b : e.a;
    e.sa_bytes = live ? s.sa_bytes : 0;
    e.sb_bytes = live ? s.sb_bytes : 0;
    return e;
}

__device__ __forceinline__ ScaleSrc scale_src(const GemmArgs& p, const TileSrc& src, int wave)
{
    const bool is_a = wave == 0, is_b = wave == 1;
    ScaleSrc c;
    c.base = is_a ? src.sa : src.sb;
    c.ld = is_a ? p.lsa : p.lsb;
    c.bytes = is_a ? src.sa_bytes : (is_b ? src.sb_bytes : 0);
    c.dst = kTileA + kTileB + (is_a ? 0 : (is_b ? 1024 : kScaleBytes));
    asm volatile("" : "+s"(c.ld));
    return c;
}

// Copy t (0 .. kOpPerWave-1) of this wave's share of a stage's A tile (op 0)
// or B tile (op 1): one 1 KiB run (8 rows of 128 bytes) of contraction block kb.
__device__ __forceinline__ void load_op_part(const GemmArgs& p, const TileSrc& src, uint8_t* stage, int kb, int wave,
                                             int lane, int t, int op)
{
    const int kcol = kb * kBK;
    const int blk = wave * kOpPerWave + t;        // 1 KiB block = 8 rows of 128 bytes
    const int ci = blk * 64 + lane;               // 16-byte chunk index within the tile
    const int row = ci >> 3;
    const int chunk = (ci & 7) ^ ((row >> 1) & 7);
    if (op == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src.a, (lds_ptr_t)(stage + blk * 1024), 16,
                                                 (uint32_t)(row * p.lda + chunk * 16), kcol, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src.b, (lds_ptr_t)(stage + kTileA + blk * 1024), 16,
                                                 (uint32_t)(row * p.ldb + chunk * 16), kcol, 0, 0);
}

// The block's scale runs: the 256 tile rows' (wave 0) and columns' (wave 1)
// scales are contiguous in the block-major layout, one 1 KiB copy each.  The
// other waves issue an empty copy into the stage's sink (no branch in the
// loop body).
__device__ __forceinline__ void load_scale_part(const ScaleSrc& sc, bool live, uint8_t* stage, int kb, int lane)
{
    const __amdgpu_buffer_rsrc_t r = make_rsrc(sc.base + kb * sc.ld, live ? sc.bytes : 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(stage + sc.dst), 16, (uint32_t)(lane * 16), 0, 0, 0);
}

// The A tile and scale copies of one stage (its B tile is copied from the
// first slots of the block before it; see block_body).
__device__ __forceinline__ void load_stage_a_scales(const GemmArgs& p, const TileSrc& src, uint8_t* stage, int kb,
                                                    int wave, int lane)
{
#pragma unroll
    for (int t = 0; t < kOpPerWave; ++t) load_op_part(p, src, stage, kb, wave, lane, t, 0);
    load_scale_part(scale_src(p, src, wave), true, stage, kb, lane);
}

// Issue all global -> LDS copies of one 128-deep stage (A tile, B tile, scales).
__device__ __forceinline__ void load_stage(const GemmArgs& p, const TileSrc& src, uint8_t* stage, int kb, int wave,
                                           int lane)
{
#pragma unroll
    for (int t = 0; t < kOpPerWave; ++t) {
        load_op_part(p, src, stage, kb, wave, lane, t, 0);
        load_op_part(p, src, stage, kb, wave, lane, t, 1);
    }
    load_scale_part(scale_src(p, src, wave), true, stage, kb, lane);
}

// This lane's byte offsets inside a stage.
struct LaneOff {
    int a_lo, a_hi;   // A fragment halves of row group 0 (row group i: + i * 2048)
    int b_lo, b_hi;   // B fragment halves of column group 0 (column group j: + j * 2048)
    int sa;           // sA of row r16 of row group 0 (+ i * 64)
    int sb_row;       // sB of column r16 of column group 0 (+ j * 64): matrix-core scale operand
    int sb_vec;       // sB of the lane's four output columns of column group 0 (+ j * 64)
};

__device__ __forceinline__ LaneOff lane_offsets(int wave, int lane)
{
    const int wm = wave / kWavesN, wn = wave % kWavesN;
    const int r16 = lane & 15, q4 = lane >> 4;
    LaneOff o;
    // adding 16 rows leaves the swizzle term unchanged, so fragment i / j is a constant offset
    o.a_lo = swz(wm * kWM + r16, q4);
    o.a_hi = swz(wm * kWM + r16, q4 + 4);
    o.b_lo = kTileA + swz(wn * kWN + r16, q4);
    o.b_hi = kTileA + swz(wn * kWN + r16, q4 + 4);
    o.sa = kTileA + kTileB + (wm * kWM + r16) * 4;
    o.sb_row = kTileA + kTileB + kBM * 4 + (wn * kWN + r16) * 4;
    o.sb_vec = kTileA + kTileB + kBM * 4 + (wn * kWN + q4 * 4) * 4;
    // Opaque to the compiler: otherwise it splits the stage-region constants
    // out of these sums and, past the 16-bit immediate offset of ds_read,
    // keeps one address register per fragment instead of one per field.
    asm volatile("" : "+v"(o.a_lo), "+v"(o.a_hi), "+v"(o.b_lo), "+v"(o.b_hi), "+v"(o.sa), "+v"(o.sb_row),
                 "+v"(o.sb_vec));
    return o;
}

// Fragment layout of the 16x16x128 fp8 operand: lane (r16, q4) holds row r16,
// bytes k = 16 q4 .. 16 q4 + 15 in registers 0-3 and k = 64 + 16 q4 .. in 4-7.
__device__ __forceinline__ void lds_half(v8i& f, int h, const uint8_t* addr)
{
    const uint4 v = *reinterpret_cast<const uint4*>(addr);
    f[4 * h + 0] = (int)v.x;
    f[4 * h + 1] = (int)v.y;
    f[4 * h + 2] = (int)v.z;
    f[4 * h + 3] = (int)v.w;
}

__device__ __forceinline__ v8i lds_frag(const uint8_t* st, int lo, int hi, int off)
{
    v8i f;
    lds_half(f, 0, st + lo + off);
    lds_half(f, 1, st + hi + off);
    return f;
}

__device__ __forceinline__ uint32_t lds_u32(const uint8_t* addr) { return *reinterpret_cast<const uint32_t*>(addr); }
__device__ __forceinline__ float lds_f32(const uint8_t* addr) { return *reinterpret_cast<const float*>(addr); }
__device__ __forceinline__ float4 lds_f32x4(const uint8_t* addr) { return *reinterpret_cast<const float4*>(addr); }

// E8M0 exponent of a positive normal power of two = its fp32 exponent field
__device__ __forceinline__ int e8m0(uint32_t bits) { return (int)(bits >> 23); }

__device__ __forceinline__ bool is_pow2_scale(float s)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, s);
    const uint32_t e = u >> 23;
    return (u & 0x007FFFFFu) == 0 && e != 0 && e < 255;  // positive normal power of two
}

// fp32 -> bf16, round to nearest even, by gfx950's v_cvt_pk_bf16_f32 (one
// instruction per pair; the integer rounding sequence costs several per value).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint16_t bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

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

// The cast's group scale and encoding with the format and power-of-two flag
// chosen at run time (the quantising epilogue; uniform branches).
__device__ __forceinline__ void quant_scale(int fmt, int pow2, float amax, float& scale, float& mult)
{
    if (fmt == FMT_E4M3) {
        if (pow2) group_scale<FMT_E4M3, true>(amax, scale, mult);
        else group_scale<FMT_E4M3, false>(amax, scale, mult);
    } else {
        if (pow2) group_scale<FMT_E5M2, true>(amax, scale, mult);
        else group_scale<FMT_E5M2, false>(amax, scale, mult);
    }
}

__device__ __forceinline__ uint2 quant_encode8(int fmt, const float (&t)[8])
{
    return fmt == FMT_E4M3 ? encode8<FMT_E4M3>(t) : encode8<FMT_E5M2>(t);
}

// The block barrier: this wave's copies have landed and its LDS reads are
// done, then every wave syncs.  No memory fence: a fenced __syncthreads()
// would also wait for copies that are meant to stay in flight.
__device__ __forceinline__ void stage_barrier()
{
    asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void promote(v4f& acc, const v4f& P, float s_a, const float4& s_b)
{
    acc[0] = fmaf(P[0], s_a * s_b.x, acc[0]);
    acc[1] = fmaf(P[1], s_a * s_b.y, acc[1]);
    acc[2] = fmaf(P[2], s_a * s_b.z, acc[2]);
    acc[3] = fmaf(P[3], s_a * s_b.w, acc[3]);
}

// Workgroup-wide AND.  Built on the kernel's own LDS array: a separate LDS
// variable (as __syncthreads_and uses) makes the compiler rewrite the alias
// scopes of every LDS access, and the stage reads would then wait for copies
// into the other stage.
__device__ __forceinline__ bool workgroup_all(bool v, uint32_t* slots, int wave, int lane)
{
    const bool w = __all(v);
    if (lane == 0) slots[wave] = w ? 1u : 0u;
    __syncthreads();
    bool r = true;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) r = r && slots[i] != 0;
    return r;
}

// A scheduling group of n LDS reads (n folds to a constant once the slot loops are unrolled).
__device__ __forceinline__ void sched_ds_reads(int n)
{
    if (n == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (n == 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    if (n == 4) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
}

// Registers a wave carries from block to block.  B column group j lives in
// slot j & 3 (streamed two groups ahead); A fragments are resident, the next
// block's copy replacing fragment i right after its last use.  Scales of the
// A rows are double-buffered by stage parity.
struct Pipe {
    v8i ac[kTM];
    v8i bq[4];
    float sa[2][kTM];     // FULL: sA values
    uint32_t ea[2][kTM];  // chain: raw sA bits
    float4 sbq[4];        // FULL: the lane's 4 sB values per column group
    uint32_t ebq[4];      // chain: raw sB bits of column r16
    v4f P[2];             // FULL: products waiting for promotion
};

// One contraction block held in stage S (`cur`); the next block is in `nxt`.
// The two come from main_loop's restrict-qualified stage pointers.
//
// Copies, one every other slot so the address unit drains them as they come
// instead of stalling the waves on a burst: right after the block's barrier
// the A tile and scales of block +2 go into `cur`; in the block's first two
// column groups the B tile of block +1 goes into `nxt` (free since the last
// barrier, and waited for at this block's barrier, ~0.6 block later).
template <int S, bool kChain, int kFmtA, int kFmtB>
__device__ __forceinline__ void block_body(const GemmArgs& p, uint8_t* cur, uint8_t* nxt,
                                           v4f (&acc)[kTM][kTN], Pipe& q, const LaneOff& o, const TileSrc& src,
                                           const ScaleSrc& sc, int kb_next1, bool has_next1, int kb_next2,
                                           bool has_next2, int wave, int lane)
{
    const TileSrc srcn1 = select_src(src, has_next1);
    const TileSrc srcn2 = select_src(src, has_next2);
    int ea[kTM];
    if (kChain) {
#pragma unroll
        for (int i = 0; i < kTM; ++i) ea[i] = e8m0(q.ea[S][i]);
    }
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
        // every read of `cur` has been issued (B groups up to 7 were read two groups ago):
        // past this barrier the copies of block +2 go into it, one per slot
        if (j == kBarrierGroup) stage_barrier();
        const int eb = kChain ? e8m0(q.ebq[j & 3]) : 0;
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
            const int t = j * kTM + i;
            if (kChain) {
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(q.bq[j & 3], q.ac[i], acc[i][j], kFmtB,
                                                                             kFmtA, 0, eb, 0, ea[i]);
            } else {
                // promote the product of two slots back (slots -2 and -1 are the previous
                // block's last two), then start this slot's product in the register it frees
                const int tp = (t + kTM * kTN - 2) % (kTM * kTN);
                const int ip = tp % kTM, jp = tp / kTM;
                promote(acc[ip][jp], q.P[t & 1], t < 2 ? q.sa[1 - S][ip] : q.sa[S][ip], q.sbq[jp & 3]);
                // pin the update to this slot (otherwise it is sunk to the end of the block and every
                // product of the block stays live)
                asm volatile("" : "+v"(acc[ip][jp]));
                q.P[t & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(q.bq[j & 3], q.ac[i],
                                                                              v4f{0.f, 0.f, 0.f, 0.f}, kFmtB, kFmtA,
                                                                              0, 0, 0, 0);
            }
            // this slot's copy into `cur` for block +2 (the A and B runs alternate; the
            // scale run rides with the first), spread so the address unit drains them
            // as they come instead of stalling the waves on a burst
            int n_vm = 0;
            if (j < 2 && (i & 1) == 0) {
                load_op_part(p, srcn1, nxt, kb_next1, wave, lane, (j * kTM + i) >> 1, 1);
                ++n_vm;
            }
            if (j >= kBarrierGroup) {
                const int c = (j - kBarrierGroup) * kTM + i;
                if ((c & 1) == 0) {
                    load_op_part(p, srcn2, cur, kb_next2, wave, lane, c >> 1, 0);
                    ++n_vm;
                } else if (c == 1) {
                    load_scale_part(sc, has_next2, cur, kb_next2, lane);
                    ++n_vm;
                }
            }
            // LDS reads of this slot
            if (j < kBarrierGroup) {
                const int jb = j + 2;  // column group prefetched from this stage
                if (i == 0) lds_half(q.bq[jb & 3], 0, cur + o.b_lo + jb * 2048);
                if (i == 1) lds_half(q.bq[jb & 3], 1, cur + o.b_hi + jb * 2048);
                if (i == 2) {
                    if (kChain) q.ebq[jb & 3] = lds_u32(cur + o.sb_row + jb * 64);
                    else q.sbq[jb & 3] = lds_f32x4(cur + o.sb_vec + jb * 64);
                }
            } else if (j == kBarrierGroup) {
                // the next block's first two column groups and its A-row scales
                if (i == 0) q.bq[0] = lds_frag(nxt, o.b_lo, o.b_hi, 0);
                if (i == 1) {
                    if (kChain) q.ebq[0] = lds_u32(nxt + o.sb_row);
                    else q.sbq[0] = lds_f32x4(nxt + o.sb_vec);
                    lds_half(q.bq[1], 0, nxt + o.b_lo + 2048);
                }
                if (i == 2) {
                    lds_half(q.bq[1], 1, nxt + o.b_hi + 2048);
                    if (kChain) q.ebq[1] = lds_u32(nxt + o.sb_row + 64);
                    else q.sbq[1] = lds_f32x4(nxt + o.sb_vec + 64);
                }
                if (i == 3) {
#pragma unroll
                    for (int r = 0; r < kTM; ++r) {
                        if (kChain) q.ea[1 - S][r] = lds_u32(nxt + o.sa + r * 64);
                        else q.sa[1 - S][r] = lds_f32(nxt + o.sa + r * 64);
                    }
                }
            } else {
                // last column group: A fragment i is dead after this slot's instruction
                q.ac[i] = lds_frag(nxt, o.a_lo, o.a_hi, i * 2048);
            }
            // Ask the scheduler for this slot's order: (FULL) the promotion of
            // the product from two slots back, the matrix-core op, then the
            // slot's LDS reads.
            const int n_ds = j < kBarrierGroup ? (i < 3 ? 1 : 0) : (j == kBarrierGroup && i == 3 ? kTM : 2);
            if (!kChain) __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (n_vm == 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            if (n_vm == 2) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
            sched_ds_reads(n_ds);
        }
    }
}

// Stage 0 of the block range has landed and stage 1 is in flight when this is
// called.  The two stages are restrict-qualified so the compiler knows the
// copies into one do not feed reads of the other and does not make those
// reads wait for them (every copy is issued from code outside this scope or
// from block_body, so none of them carries a scope the reads could alias).
template <bool kChain, int kFmtA, int kFmtB>
__device__ __forceinline__ void main_loop(const GemmArgs& p, uint8_t* __restrict__ s0, uint8_t* __restrict__ s1,
                                          v4f (&acc)[kTM][kTN], const LaneOff& o, const TileSrc& src, int kb0,
                                          int nkb, int wave, int lane)
{
    Pipe q;
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
        q.ac[i] = lds_frag(s0, o.a_lo, o.a_hi, i * 2048);
        if (kChain) q.ea[0][i] = lds_u32(s0 + o.sa + i * 64);
        else q.sa[0][i] = lds_f32(s0 + o.sa + i * 64);
        q.sa[1][i] = 0.f;
        q.ea[1][i] = 0;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        q.bq[j] = lds_frag(s0, o.b_lo, o.b_hi, j * 2048);
        if (kChain) q.ebq[j] = lds_u32(s0 + o.sb_row + j * 64);
        else q.sbq[j] = lds_f32x4(s0 + o.sb_vec + j * 64);
    }
    // the first two slots promote zero products with zero scales
    q.P[0] = q.P[1] = v4f{0.f, 0.f, 0.f, 0.f};
    q.sbq[3] = make_float4(0.f, 0.f, 0.f, 0.f);
    q.sbq[2] = q.sbq[3];
    q.ebq[2] = q.ebq[3] = 0;
    q.bq[2] = q.bq[3] = q.bq[0];

    const ScaleSrc sc = scale_src(p, src, wave);
    int it = 0;
    for (; it + 2 <= nkb; it += 2) {
        block_body<0, kChain, kFmtA, kFmtB>(p, s0, s1, acc, q, o, src, sc, kb0 + it + 1, it + 1 < nkb, kb0 + it + 2,
                                            it + 2 < nkb, wave, lane);
        block_body<1, kChain, kFmtA, kFmtB>(p, s1, s0, acc, q, o, src, sc, kb0 + it + 2, it + 2 < nkb, kb0 + it + 3,
                                            it + 3 < nkb, wave, lane);
    }
    if (it < nkb) block_body<0, kChain, kFmtA, kFmtB>(p, s0, s1, acc, q, o, src, sc, 0, false, 0, false, wave, lane);
    // the trailing copies (empty ranges) still write LDS: let them land
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (!kChain) {
        // the last two products of the last block (slots 30 and 31: registers P[0] and P[1])
        const float s_a2 = (nkb & 1) ? q.sa[0][kTM - 2] : q.sa[1][kTM - 2];
        const float s_a1 = (nkb & 1) ? q.sa[0][kTM - 1] : q.sa[1][kTM - 1];
        promote(acc[kTM - 2][kTN - 1], q.P[0], s_a2, q.sbq[(kTN - 1) & 3]);
        promote(acc[kTM - 1][kTN - 1], q.P[1], s_a1, q.sbq[(kTN - 1) & 3]);
    }
}

__device__ __forceinline__ void unpack_bf16x8(const uint4 w, float (&f)[8])
{
    f[0] = bf16_to_f32(w.x & 0xFFFF); f[1] = bf16_to_f32(w.x >> 16);
    f[2] = bf16_to_f32(w.y & 0xFFFF); f[3] = bf16_to_f32(w.y >> 16);
    f[4] = bf16_to_f32(w.z & 0xFFFF); f[5] = bf16_to_f32(w.z >> 16);
    f[6] = bf16_to_f32(w.w & 0xFFFF); f[7] = bf16_to_f32(w.w >> 16);
}

// Eight bf16 values to dst[0..7]: one 16-byte store, or element by element
// up to `left` when the run crosses the last column.
__device__ __forceinline__ void store_bf16x8(uint16_t* dst, const float (&v)[8], bool full, int64_t left)
{
    if (full) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                    pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) if (r < left) dst[r] = bf16_rne(v[r]);
    }
}

// The saved pre-activation: its reader is the backward pass, long after this
// kernel, so the full 16-byte runs are streamed (non-temporal stores: the
// forward with the pre-activation measured 3-4 % faster, the MLP training
// step 1 %); a run cut by the matrix edge goes out element by element.
// (Streamed 8-byte runs, 32 contiguous bytes per row and instruction, made
// the two-layout forward 3.5 % slower: every caller pairs column groups
// first.)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_preact_bf16x8(uint16_t* dst, const float (&v)[8], bool full, int64_t left)
{
    if (full) {
        __builtin_nontemporal_store(u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                            pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])},
                                    reinterpret_cast<u32x4_t*>(dst));
    } else {
        store_bf16x8(dst, v, full, left);
    }
}

// DPP row controls: quad_perm [1,0,3,2], [2,3,0,1], half-row mirror, row mirror.
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppRowHalfMirror = 0x141, kDppRowMirror = 0x140;

template <int kCtrl>
__device__ __forceinline__ float dpp_max(float v)
{
    const int o = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false);
    return fmaxf(v, __builtin_bit_cast(float, o));
}

// max over the 16 lanes of a DPP row (the lanes that share q4: rows r16 = 0 .. 15)
__device__ __forceinline__ float row16_max(float v)
{
    v = dpp_max<kDppQuadXor1>(v);
    v = dpp_max<kDppQuadXor2>(v);
    v = dpp_max<kDppRowHalfMirror>(v);
    return dpp_max<kDppRowMirror>(v);
}

// Four fp32 values (already scaled) -> four fp8 codes in one dword, byte t = value t.
__device__ __forceinline__ uint32_t quant_encode4(int fmt, float a, float b, float c, float d)
{
    const float fmax = fmt == FMT_E4M3 ? 448.0f : 57344.0f;
    a = __builtin_amdgcn_fmed3f(a, -fmax, fmax);
    b = __builtin_amdgcn_fmed3f(b, -fmax, fmax);
    c = __builtin_amdgcn_fmed3f(c, -fmax, fmax);
    d = __builtin_amdgcn_fmed3f(d, -fmax, fmax);
    int w;
    if (fmt == FMT_E4M3) {
        w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    } else {
        w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
        w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
    }
    return (uint32_t)w;
}

// Transposed quantising store: the tile's final values v (accumulator layout)
// cast along M in 1x128 groups, i.e. the per-token cast of the result's
// transpose (the weight gradient's along-tokens operand): qt[n][m] codes and
// qt_scales[m / 128][n].  A 128-row group is the wave pair (wm, wm ^ 1): their
// column maxima meet in LDS (region X), each lane derives the scale of 2 of
// its 32 columns and shares the multipliers through region Y; the codes of a
// column's 64 wave rows go to region T as 16 dwords (dword r16 holds rows
// 16 i + r16, byte i), then every thread takes two 64-byte runs of T,
// transposes their 4x4 byte blocks in registers and stores them as 16-byte
// runs of qt.  `xs` is a stage the epilogue may use (68 KiB).
__device__ __forceinline__ void quant_transposed(const GemmArgs& p, const v4f (&v)[kTM][kTN], int64_t m0, int64_t n0,
                                                 uint8_t* xs, int wave, int lane)
{
    // (lane-derived offsets are recomputed here: hoisted out of the tile loop
    // they would stay live across the main loop and push it into spills)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(lane), "+v"(tid));
    const int wm = wave / kWavesN, wn = wave % kWavesN;
    const int r16 = lane & 15, q4 = lane >> 4;
    float* X = reinterpret_cast<float*>(xs);          // [kWaves][kWN] column maxima
    float* Y = reinterpret_cast<float*>(xs + 4096);   // [kWaves][kWN] multipliers
    uint32_t* T = reinterpret_cast<uint32_t*>(xs);    // [kBN][kWavesM][16] code dwords (after X, Y are read)
    const int64_t mg = m0 + (wm >> 1) * 128;          // this wave pair's 128-row group
    const bool group_live = mg < p.M;                 // (M is a multiple of 128: whole groups)
    // 1. maxima of the lane's 32 columns over the wave's 64 rows
    {
        float cm[kTN][4];
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float a = fmaxf(fmaxf(fabsf(v[0][j][c]), fabsf(v[1][j][c])), fmaxf(fabsf(v[2][j][c]), fabsf(v[3][j][c])));
                cm[j][c] = row16_max(a);
            }
        if (r16 == 0) {
#pragma unroll
            for (int j = 0; j < kTN; ++j)
                *reinterpret_cast<float4*>(X + wave * kWN + j * 16 + q4 * 4) =
                    make_float4(cm[j][0], cm[j][1], cm[j][2], cm[j][3]);
        }
    }
    __syncthreads();
    // 2. two columns per lane: the group max with the partner wave's rows, the
    //    cast's scale (stored by the even wave of the pair) and multiplier
    {
        const int col = (r16 >> 1) * 16 + q4 * 4 + (r16 & 1) * 2;   // this lane's pair of the wave's 128 columns
        const float2 a = *reinterpret_cast<const float2*>(X + wave * kWN + col);
        const float2 b = *reinterpret_cast<const float2*>(X + (wave ^ kWavesN) * kWN + col);
        float s0, m0_, s1, m1_;
        quant_scale(p.q_fmt, p.q_pow2, fmaxf(a.x, b.x), s0, m0_);
        quant_scale(p.q_fmt, p.q_pow2, fmaxf(a.y, b.y), s1, m1_);
        *reinterpret_cast<float2*>(Y + wave * kWN + col) = make_float2(m0_, m1_);
        const int64_t n = n0 + wn * kWN + col;
        if ((wm & 1) == 0 && group_live && n < p.N)
            *reinterpret_cast<float2*>(p.qt_scales + (mg / 128) * p.ld_qts + n) = make_float2(s0, s1);
    }
    // (the multipliers were written by this wave: its LDS reads see them in order)
    uint32_t code[kTN][4];
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
        const float4 mu = *reinterpret_cast<const float4*>(Y + wave * kWN + j * 16 + q4 * 4);
        const float mv[4] = {mu.x, mu.y, mu.z, mu.w};
#pragma unroll
        for (int c = 0; c < 4; ++c)
            code[j][c] = quant_encode4(p.q_fmt, v[0][j][c] * mv[c], v[1][j][c] * mv[c], v[2][j][c] * mv[c],
                                       v[3][j][c] * mv[c]);
    }
    __syncthreads();   // every wave is done with X and Y
    // 3. codes into T: column n_t = wn * 128 + 16 j + 4 q4 + c, wave row block wm, dword r16
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int nt = wn * kWN + j * 16 + q4 * 4 + c;
            T[(nt * kWavesM + wm) * 16 + r16] = code[j][c];
        }
    __syncthreads();
    // 4. two 64-byte runs per thread: T[(n_t, w)] holds rows 16 i + r of the
    //    block in dword r, byte i; output dword 4 i + g takes byte i of dwords
    //    4 g .. 4 g + 3 (a 4x4 byte transpose per g)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int k = tid + h * kThreads;   // 0 .. kBN * kWavesM - 1
        const int nt = k / kWavesM, w = k % kWavesM;
        const int64_t n = n0 + nt, m = m0 + w * kWM;
        const uint4* src = reinterpret_cast<const uint4*>(T + (nt * kWavesM + w) * 16);
        uint32_t o[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint4 d = src[g];
            // [a0 b0 a1 b1], [a2 b2 a3 b3], [c0 d0 c1 d1], [c2 d2 c3 d3]
            const uint32_t ab_lo = __builtin_amdgcn_perm(d.y, d.x, 0x05010400u);
            const uint32_t ab_hi = __builtin_amdgcn_perm(d.y, d.x, 0x07030602u);
            const uint32_t cd_lo = __builtin_amdgcn_perm(d.w, d.z, 0x05010400u);
            const uint32_t cd_hi = __builtin_amdgcn_perm(d.w, d.z, 0x07030602u);
            o[0 * 4 + g] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u);
            o[1 * 4 + g] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u);
            o[2 * 4 + g] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u);
            o[3 * 4 + g] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u);
        }
        if (n < p.N && m < p.M) {
            uint8_t* dst = p.qt_out + n * p.ld_qt + m;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *reinterpret_cast<uint4*>(dst + 16 * r) = make_uint4(o[4 * r], o[4 * r + 1], o[4 * r + 2], o[4 * r + 3]);
        }
    }
}

// Row-wise quantising store from the accumulator layout: the wave's 128
// columns are one 1x128 group of each of its rows, and row 16 i + r16's
// values are the 32 held by each of the four lanes that share r16.
template <bool kFull>
__device__ __forceinline__ void quant_rowwise_acc(const GemmArgs& p, const v4f (&v)[kTM][kTN], int64_t m0, int64_t n0,
                                                  int wave, int lane)
{
    const int wm = wave / kWavesN, wn = wave % kWavesN;
    const int r16 = lane & 15, q4 = lane >> 4;
    const int64_t ng = n0 + wn * kWN;
    const bool group_in = kFull || ng < p.N;
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
        const int64_t m = m0 + wm * kWM + i * 16 + r16;
        const bool live = group_in && (kFull || m < p.M);
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) amax = fmaxf(amax, fabsf(v[i][j][c]));
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        float scale, mult;
        quant_scale(p.q_fmt, p.q_pow2, amax, scale, mult);
        uint8_t* o = p.q_out + m * p.ld_q + ng + q4 * 4;
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            const uint32_t e = quant_encode4(p.q_fmt, v[i][j][0] * mult, v[i][j][1] * mult, v[i][j][2] * mult,
                                             v[i][j][3] * mult);
            if (live) *reinterpret_cast<uint32_t*>(o + j * 16) = e;
        }
        if (live && q4 == 0) p.q_scales[(ng / 128) * p.ld_qs + m] = scale;
    }
}

// Bias gradient of columns n .. n + 3: the lane's partial column sums t
// (its rows of the wave's 64) reduced over the 16 lanes that share q4, then
// one atomic add per column, or (deterministic) one row of the workspace.
template <bool kFull>
__device__ __forceinline__ void bias_grad_cols4(const GemmArgs& p, float (&t)[4], int64_t n, int64_t m0, int wm, int r16,
                                                float* bgrad_v)
{
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        t[r] += __shfl_xor(t[r], 1);
        t[r] += __shfl_xor(t[r], 2);
        t[r] += __shfl_xor(t[r], 4);
        t[r] += __shfl_xor(t[r], 8);
    }
    if (r16 == 0 && p.bgrad_ws) {
        // deterministic: this wave's row of partial sums (the row is padded to a
        // multiple of 4 columns, so the 16-byte store never passes it)
        if (kFull || n < p.N)
            *reinterpret_cast<float4*>(p.bgrad_ws + ((m0 / kBM) * kWavesM + wm) * p.bgrad_ws_ld + n) =
                make_float4(t[0], t[1], t[2], t[3]);
    } else if (r16 == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (kFull || n + r < p.N) unsafeAtomicAdd(bgrad_v + n + r, t[r]);
    }
}

// Epilogue.  Lane (r16, q4) holds D[m][n..n+3] of every (i, j), with m = 16 i
// + r16 and n = 16 j + 4 q4 in the wave's frame.  Wgrad adds those four
// columns into out in place.  The Linear-layer epilogues pair column groups
// j, j + 1: one v_permlane16_swap per register pair exchanges the odd 16-lane
// rows of group j with the even rows of group j + 1, after which every lane
// holds eight consecutive columns of its row (group j + (q4 & 1), columns
// 8 (q4 >> 1) .. +7).  Each bf16 load and store is then a 16-byte run, and
// four lanes cover 64 contiguous bytes of a row.
template <int kEpi, bool kFull, int kQuant, int kJ = kTN>
__device__ __forceinline__ void epilogue(const GemmArgs& p, v4f (&acc)[kTM][kJ], int64_t m0, int64_t n0,
                                         int64_t out_off, const uint16_t* bias_v, float* bgrad_v, uint8_t* xs,
                                         int wave, int lane)
{
    static_assert(kJ % 2 == 0 && kJ <= kTN && (kQuant == 0 || kJ == kTN),
                  "pairs of column groups; the quantising stores take a wave's whole 128 columns");
    const int wm = wave / kWavesN, wn = wave % kWavesN;
    // (the lane index is re-derived here so that its address arithmetic is not
    // hoisted out of the tile loop and held in registers across the K loop)
    asm volatile("" : "+v"(lane));
    const int r16 = lane & 15, q4 = lane >> 4;

    // A tile inside the matrix: no bounds checks, and every load is issued
    // before the first store.  Stores count in the same vmcnt as loads, so a
    // load issued after a store cannot be waited for without also waiting for
    // that store to complete.
    if constexpr (kFull && kEpi == (int)Epi::Wgrad && kJ < kTN) {
        // A few column groups (one wave's share of the wave-tile kernel): all
        // loads in one batch, then the sums and the stores.
        float* o = reinterpret_cast<float*>(p.out) + out_off + (m0 + wm * kWM + r16) * p.ld_out + n0 + wn * kWN + q4 * 4;
        float4 c[kTM][kJ];
#pragma unroll
        for (int j = 0; j < kJ; ++j)
#pragma unroll
            for (int i = 0; i < kTM; ++i) c[i][j] = *reinterpret_cast<const float4*>(o + i * 16 * p.ld_out + j * 16);
#pragma unroll
        for (int j = 0; j < kJ; ++j)
#pragma unroll
            for (int i = 0; i < kTM; ++i) {
                const v4f& a = acc[i][j];
                float4& d = c[i][j];
                d.x += a[0]; d.y += a[1]; d.z += a[2]; d.w += a[3];
                *reinterpret_cast<float4*>(o + i * 16 * p.ld_out + j * 16) = d;
            }
        return;
    } else if constexpr (kFull && kEpi == (int)Epi::Wgrad) {
        // Four quarters of the column groups, each read in one batch and
        // added.  A quarter's loads are issued before the previous quarter's
        // stores: the load/store counter retires in issue order, so waiting
        // for those loads does not wait for the stores behind them.
        float* o = reinterpret_cast<float*>(p.out) + out_off + (m0 + wm * kWM + r16) * p.ld_out + n0 + wn * kWN + q4 * 4;
        constexpr int kQ = kTN / 4;
        float4 c[2][kTM][kQ];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
#pragma unroll
            for (int jj = 0; jj < kQ; ++jj)
#pragma unroll
                for (int i = 0; i < kTM; ++i)
                    c[h & 1][i][jj] = *reinterpret_cast<const float4*>(o + i * 16 * p.ld_out + (h * kQ + jj) * 16);
            if (h > 0) {
                // (fences for the scheduler: each quarter's loads stay after
                // the previous quarter's sums, so at most two quarters of the
                // output are held in registers besides the accumulators)
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int jj = 0; jj < kQ; ++jj)
#pragma unroll
                    for (int i = 0; i < kTM; ++i)
                        *reinterpret_cast<float4*>(o + i * 16 * p.ld_out + ((h - 1) * kQ + jj) * 16) = c[(h - 1) & 1][i][jj];
            }
#pragma unroll
            for (int jj = 0; jj < kQ; ++jj)
#pragma unroll
                for (int i = 0; i < kTM; ++i) {
                    const v4f& a = acc[i][h * kQ + jj];
                    float4& d = c[h & 1][i][jj];
                    d.x += a[0]; d.y += a[1]; d.z += a[2]; d.w += a[3];
                }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int jj = 0; jj < kQ; ++jj)
#pragma unroll
            for (int i = 0; i < kTM; ++i)
                *reinterpret_cast<float4*>(o + i * 16 * p.ld_out + (3 * kQ + jj) * 16) = c[1][i][jj];
        return;
    }

    if (kEpi == (int)Epi::Wgrad) {
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            const int64_t n = n0 + wn * kWN + j * 16 + q4 * 4;
            const bool full4 = kFull || n + 3 < p.N;
#pragma unroll
            for (int i = 0; i < kTM; ++i) {
                const int64_t m = m0 + wm * kWM + i * 16 + r16;
                if (!kFull && (m >= p.M || n >= p.N)) continue;
                float* o = reinterpret_cast<float*>(p.out) + out_off + m * p.ld_out + n;
                if (full4) {
                    float4 cur = *reinterpret_cast<float4*>(o);
                    cur.x += acc[i][j][0]; cur.y += acc[i][j][1]; cur.z += acc[i][j][2]; cur.w += acc[i][j][3];
                    *reinterpret_cast<float4*>(o) = cur;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) if (n + r < p.N) o[r] += acc[i][j][r];
                }
            }
        }
        return;
    }

    if (kEpi == (int)Epi::Dgrad) {
        // The arithmetic stays in the accumulator layout (four columns per
        // lane); the memory side uses the paired layout.  The swap is its own
        // inverse: the 16-byte run of Z a lane loads for its paired columns
        // swaps back into the bf16 pairs of its own columns, and the packed
        // results swap forward into the run it stores.  Positions past M or N
        // hold zero products (their operand rows read as zero), but a row
        // past M may carry the scale array's padding (up to three entries of
        // undefined content, copied with the 16-byte runs), so besides the
        // loads and stores the column sums skip those rows.
        const bool has_dgelu = (p.flags & TE_EPI_DGELU) != 0;
        const bool has_bgrad = (p.flags & TE_EPI_BGRAD) != 0;
        float colsum[kJ][4];
#pragma unroll
        for (int j = 0; j < kJ; ++j) colsum[j][0] = colsum[j][1] = colsum[j][2] = colsum[j][3] = 0.f;
        uint4 zq[kJ / 2][kTM];
        if (kFull && has_dgelu && !kQuant) {
#pragma unroll
            for (int jp = 0; jp < kJ / 2; ++jp)
#pragma unroll
                for (int i = 0; i < kTM; ++i)
                    zq[jp][i] = *reinterpret_cast<const uint4*>(
                        p.preact + (m0 + wm * kWM + i * 16 + r16) * p.ld_aux + n0 + wn * kWN + (2 * jp + (q4 & 1)) * 16 +
                        (q4 >> 1) * 8);
        }
        if constexpr (kQuant == 2) {
            // Both casts of D.  Pass by pass, so that each keeps only the
            // accumulator and a few registers of its own live: dGELU in place,
            // the bias gradient summed from the final values (rows in the
            // order of the row-wise path), the transposed cast, the row-wise.
            const int64_t ng = n0 + wn * kWN;
            const bool group_in = kFull || ng < p.N;
            if (has_dgelu) {
#pragma unroll
                for (int i = 0; i < kTM; ++i) {
                    const int64_t m = m0 + wm * kWM + i * 16 + r16;
                    const bool live = group_in && (kFull || m < p.M);
                    uint4 zr[kTN / 2];
#pragma unroll
                    for (int jp = 0; jp < kTN / 2; ++jp) {
                        zr[jp] = make_uint4(0u, 0u, 0u, 0u);
                        if (live)
                            zr[jp] = *reinterpret_cast<const uint4*>(
                                p.preact + m * p.ld_aux + ng + (2 * jp + (q4 & 1)) * 16 + (q4 >> 1) * 8);
                    }
#pragma unroll
                    for (int jp = 0; jp < kTN / 2; ++jp) {
                        const auto lo = __builtin_amdgcn_permlane16_swap(zr[jp].x, zr[jp].z, false, false);
                        const auto hi = __builtin_amdgcn_permlane16_swap(zr[jp].y, zr[jp].w, false, false);
                        const uint32_t a0 = lo[0], b0 = lo[1], a1 = hi[0], b1 = hi[1];
                        v4f& v0 = acc[i][2 * jp];
                        v4f& v1 = acc[i][2 * jp + 1];
                        v0[0] *= dgelu(bf16_to_f32(a0 & 0xFFFF)); v0[1] *= dgelu(bf16_to_f32(a0 >> 16));
                        v0[2] *= dgelu(bf16_to_f32(a1 & 0xFFFF)); v0[3] *= dgelu(bf16_to_f32(a1 >> 16));
                        v1[0] *= dgelu(bf16_to_f32(b0 & 0xFFFF)); v1[1] *= dgelu(bf16_to_f32(b0 >> 16));
                        v1[2] *= dgelu(bf16_to_f32(b1 & 0xFFFF)); v1[3] *= dgelu(bf16_to_f32(b1 >> 16));
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if (has_bgrad) {
#pragma unroll
                for (int j = 0; j < kTN; ++j) {
                    float t[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < kTM; ++i)
                        if (kFull || m0 + wm * kWM + i * 16 + r16 < p.M) {
#pragma unroll
                            for (int c = 0; c < 4; ++c) t[c] += acc[i][j][c];
                        }
                    bias_grad_cols4<kFull>(p, t, ng + j * 16 + q4 * 4, m0, wm, r16, bgrad_v);
                }
            }
            quant_transposed(p, acc, m0, n0, xs, wave, lane);
            if (p.q_out) quant_rowwise_acc<kFull>(p, acc, m0, n0, wave, lane);
            return;
        }
        if constexpr (kQuant != 0) {
            // Quantising store of D (after dGELU): as in the forward, the
            // wave's 128 columns are one 1x128 group of each row; the lane's
            // 32 values of a row are its 8 column groups x 4 columns.
            const int64_t ng = n0 + wn * kWN;
            const bool group_in = kFull || ng < p.N;
#pragma unroll
            for (int i = 0; i < kTM; ++i) {
                const int64_t m = m0 + wm * kWM + i * 16 + r16;
                const bool live = group_in && (kFull || m < p.M);
                float v[kTN][4];
#pragma unroll
                for (int j = 0; j < kTN; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c) v[j][c] = acc[i][j][c];
                if (has_dgelu) {
                    // (this row's four Z runs, loaded together; the whole tile's
                    // runs do not fit in registers beside the row's values)
                    uint4 zr[kTN / 2];
#pragma unroll
                    for (int jp = 0; jp < kTN / 2; ++jp) {
                        zr[jp] = make_uint4(0u, 0u, 0u, 0u);
                        if (live)
                            zr[jp] = *reinterpret_cast<const uint4*>(
                                p.preact + m * p.ld_aux + ng + (2 * jp + (q4 & 1)) * 16 + (q4 >> 1) * 8);
                    }
#pragma unroll
                    for (int jp = 0; jp < kTN / 2; ++jp) {
                        const uint32_t zw[4] = {zr[jp].x, zr[jp].y, zr[jp].z, zr[jp].w};
                        const auto lo = __builtin_amdgcn_permlane16_swap(zw[0], zw[2], false, false);
                        const auto hi = __builtin_amdgcn_permlane16_swap(zw[1], zw[3], false, false);
                        const uint32_t a0 = lo[0], b0 = lo[1], a1 = hi[0], b1 = hi[1];
                        float* v0 = v[2 * jp];
                        float* v1 = v[2 * jp + 1];
                        v0[0] *= dgelu(bf16_to_f32(a0 & 0xFFFF)); v0[1] *= dgelu(bf16_to_f32(a0 >> 16));
                        v0[2] *= dgelu(bf16_to_f32(a1 & 0xFFFF)); v0[3] *= dgelu(bf16_to_f32(a1 >> 16));
                        v1[0] *= dgelu(bf16_to_f32(b0 & 0xFFFF)); v1[1] *= dgelu(bf16_to_f32(b0 >> 16));
                        v1[2] *= dgelu(bf16_to_f32(b1 & 0xFFFF)); v1[3] *= dgelu(bf16_to_f32(b1 >> 16));
                    }
                }
                float amax = 0.0f;
#pragma unroll
                for (int j = 0; j < kTN; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        if (has_bgrad && (kFull || m < p.M)) colsum[j][c] += v[j][c];
                        amax = fmaxf(amax, fabsf(v[j][c]));
                    }
                if (p.q_out) {
                    amax = fmaxf(amax, __shfl_xor(amax, 16));
                    amax = fmaxf(amax, __shfl_xor(amax, 32));
                    float scale, mult;
                    quant_scale(p.q_fmt, p.q_pow2, amax, scale, mult);
#pragma unroll
                    for (int jp = 0; jp < kTN / 2; ++jp) {
                        float t[8];
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            t[c] = v[2 * jp][c] * mult;
                            t[4 + c] = v[2 * jp + 1][c] * mult;
                        }
                        const uint2 e = quant_encode8(p.q_fmt, t);
                        if (live) {
                            uint8_t* o = p.q_out + m * p.ld_q + ng + q4 * 4;
                            *reinterpret_cast<uint32_t*>(o + (2 * jp) * 16) = e.x;
                            *reinterpret_cast<uint32_t*>(o + (2 * jp + 1) * 16) = e.y;
                        }
                    }
                    if (live && q4 == 0) p.q_scales[(ng / 128) * p.ld_qs + m] = scale;
                }
                // (one row at a time: keeps the next rows' Z loads and values out of this row's registers)
                __builtin_amdgcn_sched_barrier(0);
            }
        } else
#pragma unroll
        for (int jp = 0; jp < kJ / 2; ++jp) {
            const int j0 = 2 * jp, j1 = 2 * jp + 1;
            const int64_t np = n0 + wn * kWN + (j0 + (q4 & 1)) * 16 + (q4 >> 1) * 8;  // this lane's run
            const bool fullp = kFull || np + 7 < p.N;
#pragma unroll
            for (int i = 0; i < kTM; ++i) {
                const int64_t m = m0 + wm * kWM + i * 16 + r16;
                const bool live = kFull || (m < p.M && np < p.N);
                float v0[4] = {acc[i][j0][0], acc[i][j0][1], acc[i][j0][2], acc[i][j0][3]};
                float v1[4] = {acc[i][j1][0], acc[i][j1][1], acc[i][j1][2], acc[i][j1][3]};
                if (has_dgelu) {
                    uint32_t zw[4] = {0u, 0u, 0u, 0u};
                    const uint16_t* z = p.preact + m * p.ld_aux + np;
                    if (kFull) {
                        zw[0] = zq[jp][i].x; zw[1] = zq[jp][i].y; zw[2] = zq[jp][i].z; zw[3] = zq[jp][i].w;
                    } else if (live && fullp) {
                        const uint4 t = *reinterpret_cast<const uint4*>(z);
                        zw[0] = t.x; zw[1] = t.y; zw[2] = t.z; zw[3] = t.w;
                    } else if (live) {
#pragma unroll
                        for (int r = 0; r < 8; ++r)
                            if (np + r < p.N) zw[r >> 1] |= (uint32_t)z[r] << (16 * (r & 1));
                    }
                    const auto lo = __builtin_amdgcn_permlane16_swap(zw[0], zw[2], false, false);
                    const auto hi = __builtin_amdgcn_permlane16_swap(zw[1], zw[3], false, false);
                    const uint32_t a0 = lo[0], b0 = lo[1], a1 = hi[0], b1 = hi[1];
                    v0[0] *= dgelu(bf16_to_f32(a0 & 0xFFFF)); v0[1] *= dgelu(bf16_to_f32(a0 >> 16));
                    v0[2] *= dgelu(bf16_to_f32(a1 & 0xFFFF)); v0[3] *= dgelu(bf16_to_f32(a1 >> 16));
                    v1[0] *= dgelu(bf16_to_f32(b0 & 0xFFFF)); v1[1] *= dgelu(bf16_to_f32(b0 >> 16));
                    v1[2] *= dgelu(bf16_to_f32(b1 & 0xFFFF)); v1[3] *= dgelu(bf16_to_f32(b1 >> 16));
                }
                if (has_bgrad && (kFull || m < p.M)) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        colsum[j0][r] += v0[r];
                        colsum[j1][r] += v1[r];
                    }
                }
                if (p.out_bf16) {
                    const auto lo = __builtin_amdgcn_permlane16_swap(pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v1[0], v1[1]),
                                                                     false, false);
                    const auto hi = __builtin_amdgcn_permlane16_swap(pack_bf16x2(v0[2], v0[3]), pack_bf16x2(v1[2], v1[3]),
                                                                     false, false);
                    uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + out_off + m * p.ld_out + np;
                    const uint32_t w[4] = {(uint32_t)lo[0], (uint32_t)hi[0], (uint32_t)lo[1], (uint32_t)hi[1]};
                    if (live && fullp) {
                        *reinterpret_cast<uint4*>(o) = make_uint4(w[0], w[1], w[2], w[3]);
                    } else if (live) {
#pragma unroll
                        for (int r = 0; r < 8; ++r)
                            if (np + r < p.N) o[r] = (uint16_t)(w[r >> 1] >> (16 * (r & 1)));
                    }
                } else {
                    // fp32: the accumulator layout already gives 16-byte runs
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const float* v = h ? v1 : v0;
                        const int64_t n = n0 + wn * kWN + (j0 + h) * 16 + q4 * 4;
                        if (!kFull && (m >= p.M || n >= p.N)) continue;
                        float* o = reinterpret_cast<float*>(p.out) + out_off + m * p.ld_out + n;
                        if (kFull || n + 3 < p.N) {
                            *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r) if (n + r < p.N) o[r] = v[r];
                        }
                    }
                }
            }
        }
        if (has_bgrad) {
#pragma unroll
            for (int j = 0; j < kJ; ++j)
                bias_grad_cols4<kFull>(p, colsum[j], n0 + wn * kWN + j * 16 + q4 * 4, m0, wm, r16, bgrad_v);
        }
        return;
    }

    // forward: pair column groups so that each lane owns eight consecutive columns
    const bool has_bias = (p.flags & TE_EPI_BIAS) != 0;
    const bool has_gelu = (p.flags & TE_EPI_GELU) != 0;
    const bool has_aux = (p.flags & TE_EPI_AUX_PREACT) != 0;
    uint4 bw[kJ / 2];

    if constexpr (kQuant == 2) {
        // Both casts of the result.  The final values are formed in place in
        // the accumulator layout (bias, pre-activation store, GELU), then the
        // transposed and the row-wise casts read them; each pass keeps only
        // the accumulator and a few registers of its own live.
        const int64_t ng = n0 + wn * kWN;
        const bool group_in = kFull || ng < p.N;
        uint2 bj[kTN];   // the bias of the lane's four columns of each group, bf16
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            bj[j] = make_uint2(0u, 0u);
            if (has_bias && group_in) bj[j] = *reinterpret_cast<const uint2*>(bias_v + ng + j * 16 + q4 * 4);
        }
        // (one flag at a time over whole accumulator vectors: a vector updated
        // element by element under per-element branches is copied and spilled)
        if (has_bias) {
#pragma unroll
            for (int j = 0; j < kTN; ++j) {
                const v4f b = {__uint_as_float(bj[j].x << 16), __uint_as_float(bj[j].x & 0xFFFF0000u),
                               __uint_as_float(bj[j].y << 16), __uint_as_float(bj[j].y & 0xFFFF0000u)};
#pragma unroll
                for (int i = 0; i < kTM; ++i) acc[i][j] += b;
            }
        }
        if (has_aux) {
            // (paired column groups, as in the other forward epilogues: 16-byte runs, streamed)
#pragma unroll
            for (int i = 0; i < kTM; ++i) {
                const int64_t m = m0 + wm * kWM + i * 16 + r16;
                const bool live = group_in && (kFull || m < p.M);
#pragma unroll
                for (int jp = 0; jp < kTN / 2; ++jp) {
                    float v[8];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const auto sw = __builtin_amdgcn_permlane16_swap(
                            __float_as_uint(acc[i][2 * jp][c]), __float_as_uint(acc[i][2 * jp + 1][c]), false, false);
                        v[c] = __uint_as_float(sw[0]);
                        v[4 + c] = __uint_as_float(sw[1]);
                    }
                    if (live)
                        store_preact_bf16x8(p.aux + m * p.ld_aux + ng + (2 * jp + (q4 & 1)) * 16 + (q4 >> 1) * 8, v,
                                            true, 8);
                }
            }
        }
        if (has_gelu) {
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int j = 0; j < kTN; ++j) {
                    const v4f t = acc[i][j];
                    acc[i][j] = v4f{gelu(t[0]), gelu(t[1]), gelu(t[2]), gelu(t[3])};
                }
        }
        quant_transposed(p, acc, m0, n0, xs, wave, lane);
        if (p.q_out) quant_rowwise_acc<kFull>(p, acc, m0, n0, wave, lane);
        return;
    }
    if constexpr (kQuant != 0) {
        // Quantising store.  A wave's 128 columns are one 1x128 group of each
        // of its rows (N is a multiple of 128, tile corners of 256), so a
        // group is wholly inside or outside the matrix, and a row's amax is
        // the max over the lane's 32 values and the 4 lanes sharing r16.
        const int64_t ng = n0 + wn * kWN;
        const bool group_in = kFull || ng < p.N;
#pragma unroll
        for (int jp = 0; jp < kTN / 2; ++jp) {
            bw[jp] = make_uint4(0u, 0u, 0u, 0u);
            if (has_bias && group_in)
                bw[jp] = *reinterpret_cast<const uint4*>(bias_v + ng + (2 * jp + (q4 & 1)) * 16 + (q4 >> 1) * 8);
        }
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
            const int64_t m = m0 + wm * kWM + i * 16 + r16;
            const bool live = group_in && (kFull || m < p.M);
            float v[kTN / 2][8];
#pragma unroll
            for (int jp = 0; jp < kTN / 2; ++jp) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const auto sw = __builtin_amdgcn_permlane16_swap(
                        __float_as_uint(acc[i][2 * jp][c]), __float_as_uint(acc[i][2 * jp + 1][c]), false, false);
                    v[jp][c] = __uint_as_float(sw[0]);
                    v[jp][4 + c] = __uint_as_float(sw[1]);
                }
                const int64_t n = ng + (2 * jp + (q4 & 1)) * 16 + (q4 >> 1) * 8;
                if (has_bias) {
                    float b8[8];
                    unpack_bf16x8(bw[jp], b8);
#pragma unroll
                    for (int r = 0; r < 8; ++r) v[jp][r] += b8[r];
                }
                if (has_aux && live) store_preact_bf16x8(p.aux + m * p.ld_aux + n, v[jp], true, 8);
                if (has_gelu) {
#pragma unroll
                    for (int r = 0; r < 8; ++r) v[jp][r] = gelu(v[jp][r]);
                }
            }
            if (p.q_out) {
                float amax = 0.0f;
#pragma unroll
                for (int jp = 0; jp < kTN / 2; ++jp)
#pragma unroll
                    for (int r = 0; r < 8; ++r) amax = fmaxf(amax, fabsf(v[jp][r]));
                amax = fmaxf(amax, __shfl_xor(amax, 16));
                amax = fmaxf(amax, __shfl_xor(amax, 32));
                float scale, mult;
                quant_scale(p.q_fmt, p.q_pow2, amax, scale, mult);
#pragma unroll
                for (int jp = 0; jp < kTN / 2; ++jp) {
                    float t[8];
#pragma unroll
                    for (int r = 0; r < 8; ++r) t[r] = v[jp][r] * mult;
                    const uint2 c = quant_encode8(p.q_fmt, t);
                    const int64_t n = ng + (2 * jp + (q4 & 1)) * 16 + (q4 >> 1) * 8;
                    if (live) *reinterpret_cast<uint2*>(p.q_out + m * p.ld_q + n) = c;
                }
                if (live && q4 == 0) p.q_scales[(ng / 128) * p.ld_qs + m] = scale;
            }
        }
        return;
    }

    if (kFull && has_bias) {
#pragma unroll
        for (int jp = 0; jp < kJ / 2; ++jp)
            bw[jp] = *reinterpret_cast<const uint4*>(bias_v + n0 + wn * kWN + (2 * jp + (q4 & 1)) * 16 + (q4 >> 1) * 8);
    }
#pragma unroll
    for (int jp = 0; jp < kJ / 2; ++jp) {
        const int64_t n = n0 + wn * kWN + (2 * jp + (q4 & 1)) * 16 + (q4 >> 1) * 8;
        const bool full8 = kFull || n + 7 < p.N;
        float bias[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (has_bias) {
            if (kFull) {
                unpack_bf16x8(bw[jp], bias);
            } else if (full8) {
                unpack_bf16x8(*reinterpret_cast<const uint4*>(bias_v + n), bias);
            } else {
#pragma unroll
                for (int r = 0; r < 8; ++r) if (n + r < p.N) bias[r] = bf16_to_f32(bias_v[n + r]);
            }
        }
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
            // (every lane takes part in the swap, before any lane drops out;
            // __float_as_uint, not __builtin_bit_cast, which reads element 0
            // when handed an element of a vector register)
            float v[8];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[i][2 * jp][c]),
                                                                 __float_as_uint(acc[i][2 * jp + 1][c]), false, false);
                v[c] = __uint_as_float(sw[0]);
                v[4 + c] = __uint_as_float(sw[1]);
            }
            const int64_t m = m0 + wm * kWM + i * 16 + r16;
            if (!kFull && (m >= p.M || n >= p.N)) continue;
#pragma unroll
            for (int r = 0; r < 8; ++r) v[r] += bias[r];
            if (has_aux) store_preact_bf16x8(p.aux + m * p.ld_aux + n, v, full8, p.N - n);
            if (has_gelu) {
#pragma unroll
                for (int r = 0; r < 8; ++r) v[r] = gelu(v[r]);
            }
            if (p.out_bf16) {
                store_bf16x8(reinterpret_cast<uint16_t*>(p.out) + out_off + m * p.ld_out + n, v, full8, p.N - n);
            } else {
                float* o = reinterpret_cast<float*>(p.out) + out_off + m * p.ld_out + n;
                if (full8) {
                    reinterpret_cast<float4*>(o)[0] = make_float4(v[0], v[1], v[2], v[3]);
                    reinterpret_cast<float4*>(o)[1] = make_float4(v[4], v[5], v[6], v[7]);
                } else {
#pragma unroll
                    for (int r = 0; r < 8; ++r) if (n + r < p.N) o[r] = v[r];
                }
            }
        }
    }
}

// One output tile: its corner, contraction range and output matrix.
struct TileCtx {
    int64_t m0, n0, out_off;
    int64_t bgrp;  // expert of an M-grouped tile (0 otherwise)
    int kb0, nkb;
    TileSrc src;
};

// Tiles of a group are rastered in bands of at most kGroupM tile rows, column
// by column inside a band, so the tiles in flight at once share A rows and B
// columns.  The rows are spread evenly over the bands (28 tile rows: four
// bands of 7, not 8 + 8 + 8 + 4), so that the run of consecutive tiles one XCD
// takes stays inside one band: the 7168 x 2112 weight gradient then fetches
// 173 MB per launch instead of 193.
__device__ __forceinline__ TileCtx tile_ctx(const GemmArgs& p, int64_t tile)
{
    const int64_t tiles_m = (p.M + kBM - 1) / kBM;
    const int64_t tiles_n = (p.N + kBN - 1) / kBN;
    const int64_t tiles_per_group = tiles_m * tiles_n;
    const int gslot = (int)(tile / tiles_per_group);
    int64_t t = tile - (int64_t)gslot * tiles_per_group;
    const int bands = (int)((tiles_m + kGroupM - 1) / kGroupM);
    const int group_m = (int)((tiles_m + bands - 1) / bands);
    const int64_t per_band = (int64_t)group_m * tiles_n;
    const int64_t band = t / per_band;
    const int64_t first_m = band * group_m;
    const int64_t band_rows = min((int64_t)group_m, tiles_m - first_m);
    t -= band * per_band;
    Group grp;
    if (p.group_k_dev) {
        // group sizes in device memory: the range of group gslot starts after
        // the earlier groups; every offset and length is clamped to the
        // operands' sum_kb blocks, so no value can move a read outside them
        int64_t off = 0;
        for (int h = 0; h < gslot; ++h) off += max(p.group_k_dev[h], (int64_t)0) / kBK;
        off = min(off, p.sum_kb);
        const int64_t len = min(max(p.group_k_dev[gslot], (int64_t)0) / kBK, p.sum_kb - off);
        grp = Group{(int32_t)off, (int32_t)len, gslot, 0};
    } else {
        grp = p.groups[gslot];
    }
    TileCtx c;
    c.m0 = (first_m + t % band_rows) * kBM;
    c.n0 = (t / band_rows) * kBN;
    c.out_off = (int64_t)grp.out_idx * p.out_group_stride;
    c.kb0 = grp.kb_off;
    c.nkb = grp.kb_len;
    c.bgrp = 0;
    if (p.m_block_group) {
        const int32_t e = p.m_block_group[c.m0 / kMGroupRows];
        if (e >= 0 && e < p.num_b_groups) c.bgrp = e;
        else c.nkb = 0;
    }
    // an empty group's or a skipped block's tile copies nothing and leaves its output untouched
    c.src = select_src(tile_src(p, c.m0, c.n0, c.bgrp), c.nkb > 0);
    return c;
}

// This thread's share of the FAST test: are the scales of the tile's rows (A)
// and columns (B) over its contraction range all powers of two?  Per block the
// tile has 2 x 64 runs of four consecutive scales (16-byte aligned: tile
// corners are multiples of 256, the leading dimension a multiple of 4); thread
// t takes runs t, t + 512, ... eight at a time, so its loads are in flight
// together.  Scales past the last row or column (the padding up to the leading
// dimension) are ignored.
__device__ __forceinline__ bool row_scales_pow2(const GemmArgs& p, const TileCtx& c)
{
    const int t = threadIdx.x;
    const int runs = c.nkb * 2 * (kBM / 4);
    bool ok = true;
    for (int f0 = 0; f0 < runs; f0 += kThreads * 8) {
        float4 v[8];
        int64_t left[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int f = f0 + u * kThreads + t;
            const int kb = c.kb0 + (f >> 7), w = f & 127;
            const bool is_a = w < kBM / 4;
            const int64_t r = (int64_t)(w & (kBM / 4 - 1)) * 4;
            left[u] = f < runs ? (is_a ? p.M - c.m0 : p.N - c.n0) - r : 0;
            v[u] = make_float4(1.f, 1.f, 1.f, 1.f);
            if (left[u] > 0)
                v[u] = *reinterpret_cast<const float4*>(is_a ? p.sa + (int64_t)kb * p.lsa + c.m0 + r
                                                             : p.sb + c.bgrp * p.sb_group_stride +
                                                                   (int64_t)kb * p.lsb + c.n0 + r);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            ok = ok && is_pow2_scale(v[u].x) && (left[u] < 2 || is_pow2_scale(v[u].y)) &&
                 (left[u] < 3 || is_pow2_scale(v[u].z)) && (left[u] < 4 || is_pow2_scale(v[u].w));
        }
    }
    return ok;
}

// Persistent kernel: workgroup w takes tiles w, w + G, w + 2G, ... (G = grid
// size).  While a tile's epilogue runs, the first stage of the workgroup's
// next tile is already being copied in; the next tile's FAST test follows the
// epilogue.
template <int kFmtA, int kFmtB, bool kFast, int kEpi, int kQuant>
__global__ __launch_bounds__(kThreads) void gemm_nt_kernel(const GemmArgs p, int64_t total_tiles)
{
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStageBytes + kWaves * 4];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // Workgroups are handed to the eight XCDs round-robin; renumber them so
    // that the tiles one XCD runs at the same time are neighbours (each XCD
    // has its own L2).
    const int64_t G = gridDim.x;
    const int64_t per_xcd = G / kXcds;
    int64_t tile = blockIdx.x;
    if (tile < per_xcd * kXcds) tile = (tile % kXcds) * per_xcd + tile / kXcds;

    const LaneOff o = lane_offsets(wave, lane);
    // (Both stage offsets are hidden: a pointer the compiler can fold to a
    // constant loses its restrict scope once main_loop is inlined.)
    int s0_off = 0, s1_off = kStageBytes;
    asm volatile("" : "+s"(s0_off), "+s"(s1_off));
    uint32_t* slots = reinterpret_cast<uint32_t*>(smem + 2 * kStageBytes);

    TileCtx c = tile_ctx(p, tile);
    load_stage(p, c.src, smem + s0_off, c.kb0, wave, lane);
    bool ok = kFast ? row_scales_pow2(p, c) : false;
    for (;;) {
        // The scaled matrix-core chain is exact only for power-of-two scales:
        // take it when every scale of this tile's rows and columns over the
        // contraction range is one.
        const bool chain = kFast && workgroup_all(ok, slots, wave, lane);
        stage_barrier();
        // (the B tile of this stage follows from the first block's first slots)
        load_stage_a_scales(p, select_src(c.src, c.nkb > 1), smem + s1_off, c.kb0 + 1, wave, lane);

        v4f acc[kTM][kTN];
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int j = 0; j < kTN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        if (chain) {
            main_loop<true, kFmtA, kFmtB>(p, smem + s0_off, smem + s1_off, acc, o, c.src, c.kb0, c.nkb, wave, lane);
        } else {
            main_loop<false, kFmtA, kFmtB>(p, smem + s0_off, smem + s1_off, acc, o, c.src, c.kb0, c.nkb, wave, lane);
        }

        // every wave is done reading the stages: start the next tile's copies
        // (and its scale test), then write this tile out
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const int64_t next = tile + G;
        const bool more = next < total_tiles;
        TileCtx cn = c;
        if (more) {
            cn = tile_ctx(p, next);
            load_stage(p, cn.src, smem + s0_off, cn.kb0, wave, lane);
        }
        // (a tile inside the matrix takes the copy of the epilogue without
        // bounds checks: straight-line code lets its loads be in flight together)
        if (c.nkb > 0) {
            // an expert's bias and bias gradient (M-grouped; offset 0 otherwise)
            const uint16_t* bias_v = p.bias + c.bgrp * p.bias_group_stride;
            float* bgrad_v = p.bias_grad + c.bgrp * p.bias_group_stride;
            // (the stage the next tile's first copies do not use is free during the
            // epilogue; the quantising stores keep one copy, with bounds checks: given
            // two copies of their long epilogues the register allocator spills in one)
            if (kQuant == 0 && c.m0 + kBM <= p.M && c.n0 + kBN <= p.N)
                epilogue<kEpi, kQuant == 0, kQuant>(p, acc, c.m0, c.n0, c.out_off, bias_v, bgrad_v, smem + s1_off,
                                                    wave, lane);
            else
                epilogue<kEpi, false, kQuant>(p, acc, c.m0, c.n0, c.out_off, bias_v, bgrad_v, smem + s1_off, wave,
                                              lane);
        }
        if (!more) break;
        // (after the epilogue: the scale reads overlap its stores)
        if (kFast) ok = row_scales_pow2(p, cn);
        tile = next;
        c = cn;
    }
}

// ---------------------------------------------------------------------------
// Wave-tile path, for GEMMs with few 256 x 256 tiles (the persistent kernel
// would leave most compute units idle: one 256 x 256 x 512 product runs on
// one of 256).  Each workgroup computes one wave tile (64 rows x 128 columns)
// of the same tile grid, so the eight wave tiles of a tile run on up to eight
// compute units, with four waves, one per SIMD: wave w runs the products of
// column groups 2w and 2w + 1 of every block from three LDS stages the four
// share.  After the K loop each wave runs the Linear-layer and weight-
// gradient epilogues on its own two column groups (a pair, the unit those
// epilogues work on); the quantising stores, whose 1 x 128 groups span the
// wave tile's 128 columns, take the four waves' accumulators in wave 0
// through LDS.  Either way the epilogue sees the wave tile's place in its
// tile.  Fragments, promotion order, matrix-core chain and epilogue are the
// persistent kernel's, so both paths give the same bits wherever the chain
// decision agrees (the persistent kernel takes it per 256 x 256 tile, this
// path per wave tile).
constexpr int kVA = kWM * kBK;                         // 8 KiB: the wave tile's A rows of one block
constexpr int kVB = kWN * kBK;                         // 16 KiB: its B rows
constexpr int kVScale = kVA + kVB;                     // sA run (1 KiB copy, 64 floats used), then sB's
constexpr int kVStage = kVA + kVB + 2 * 1024;          // 26 KiB
constexpr int kVStages = 3;
constexpr int kVCopies = kVA / 1024 + kVB / 1024 + 2;  // copies per block: 8 A + 16 B + 2 scale runs
constexpr int kVWaves = 4;                             // waves of a workgroup (one per SIMD)
constexpr int kVJ = kTN / kVWaves;                     // column groups per wave (2)
constexpr int kVThreads = 64 * kVWaves;

struct WaveSrc {
    __amdgpu_buffer_rsrc_t a, b;
    const float* sa;   // the wave tile's first row in block 0 of the block-major scales
    const float* sb;
    int sa_bytes, sb_bytes;
};

// Wave w's share of one block's copies into a stage: copies w, w + 4, ...
// (7 for waves 0 and 1, 6 for waves 2 and 3; empty ranges when `live` is
// false, so each wave's count per block stays fixed, which the waits rely on).
__device__ __forceinline__ void wave_load_part(const GemmArgs& p, const WaveSrc& s, uint8_t* stage, int kb, bool live,
                                               int w, int lane)
{
    const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(nullptr, 0, 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t ra = live ? s.a : none, rb = live ? s.b : none;
    const int kcol = live ? kb * kBK : 0;
    const int64_t kbl = live ? kb : 0;
#pragma unroll
    for (int u = 0; u < (kVCopies + kVWaves - 1) / kVWaves; ++u) {
        const int t = w + kVWaves * u;
        if (t < kVA / 1024) {
            const int ci = t * 64 + lane, row = ci >> 3, chunk = (ci & 7) ^ ((row >> 1) & 7);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(stage + t * 1024), 16,
                                                     (uint32_t)(row * p.lda + chunk * 16), kcol, 0, 0);
        } else if (t < (kVA + kVB) / 1024) {
            const int tb = t - kVA / 1024;
            const int ci = tb * 64 + lane, row = ci >> 3, chunk = (ci & 7) ^ ((row >> 1) & 7);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(stage + kVA + tb * 1024), 16,
                                                     (uint32_t)(row * p.ldb + chunk * 16), kcol, 0, 0);
        } else if (t == (kVA + kVB) / 1024) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(s.sa + kbl * p.lsa, live ? s.sa_bytes : 0),
                                                     (lds_ptr_t)(stage + kVScale), 16, (uint32_t)(lane * 16), 0, 0,
                                                     0);
        } else if (t == (kVA + kVB) / 1024 + 1) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(s.sb + kbl * p.lsb, live ? s.sb_bytes : 0),
                                                     (lds_ptr_t)(stage + kVScale + 1024), 16, (uint32_t)(lane * 16),
                                                     0, 0, 0);
        }
    }
}

// Every scale of the wave tile's rows and columns over the contraction range
// is a power of two (rows past M and columns past N do not count).
__device__ __forceinline__ bool wave_scales_pow2(const GemmArgs& p, const WaveSrc& s, int64_t m0, int64_t n0,
                                                 int kb0, int nkb, int lane)
{
    const int rows = (int)min((int64_t)kWM, p.M - m0), cols = (int)min((int64_t)kWN, p.N - n0);
    bool ok = true;
    for (int kb = kb0; kb < kb0 + nkb; ++kb) {
        const float* a = s.sa + (int64_t)kb * p.lsa;
        const float* b = s.sb + (int64_t)kb * p.lsb;
        if (lane < rows) ok = ok && is_pow2_scale(a[lane]);
        if (lane < cols) ok = ok && is_pow2_scale(b[lane]);
        if (lane + 64 < cols) ok = ok && is_pow2_scale(b[lane + 64]);
    }
    return __builtin_amdgcn_ballot_w64(!ok) == 0;
}

struct WaveLane {
    int a_lo, a_hi, b_lo, b_hi;   // fragment offsets in a stage (row group i / column group j: + 2048 each)
    int r16, q4;
};

// One block from stage `st`: wait for this wave's copies of it, meet the other
// waves (everyone's copies have landed and everyone is done with the stage of
// the block before, `nx`), refill `nx` with block kb_refill, then this wave's
// products of the block (its two column groups; promoted, or chained on
// power-of-two scales).
template <bool kChain, int kFmtA, int kFmtB>
__device__ __forceinline__ void wave_block(const GemmArgs& p, const WaveSrc& s, uint8_t* st, uint8_t* nx,
                                           v4f (&acc)[kTM][kVJ], const WaveLane& o, int w, int kb_refill, bool refill,
                                           int lane)
{
    // (the next block's copies, issued after this block's, may stay in flight)
    if (w < 2) asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    asm volatile("s_barrier" ::: "memory");
    wave_load_part(p, s, nx, kb_refill, refill, w, lane);
    v8i ac[kTM];
    float sa[kTM];
    int ea[kTM];
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
        ac[i] = lds_frag(st, o.a_lo, o.a_hi, i * 2048);
        const uint32_t bits = lds_u32(st + kVScale + (i * 16 + o.r16) * 4);
        sa[i] = __builtin_bit_cast(float, bits);
        ea[i] = e8m0(bits);
    }
#pragma unroll
    for (int jj = 0; jj < kVJ; ++jj) {
        const int j = w * kVJ + jj;
        const v8i bq = lds_frag(st, o.b_lo, o.b_hi, j * 2048);
        if (kChain) {
            const int eb = e8m0(lds_u32(st + kVScale + 1024 + (j * 16 + o.r16) * 4));
#pragma unroll
            for (int i = 0; i < kTM; ++i)
                acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bq, ac[i], acc[i][jj], kFmtB, kFmtA, 0,
                                                                              eb, 0, ea[i]);
        } else {
            const float4 sbq = lds_f32x4(st + kVScale + 1024 + (j * 16 + o.q4 * 4) * 4);
#pragma unroll
            for (int i = 0; i < kTM; ++i) {
                const v4f P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bq, ac[i], v4f{0.f, 0.f, 0.f, 0.f},
                                                                               kFmtB, kFmtA, 0, 0, 0, 0);
                promote(acc[i][jj], P, sa[i], sbq);
            }
        }
    }
}

// The K loop over three stages, unrolled by three so that each stage is its
// own restrict-qualified pointer: reads of one stage then wait only for the
// copies into that stage, not for the block in flight behind them.  Blocks 0
// and 1 are in stages 0 and 1 on entry.
template <bool kChain, int kFmtA, int kFmtB>
__device__ __forceinline__ void wave_main_loop(const GemmArgs& p, const WaveSrc& s, uint8_t* __restrict__ s0,
                                               uint8_t* __restrict__ s1, uint8_t* __restrict__ s2,
                                               v4f (&acc)[kTM][kVJ], const WaveLane& o, int w, int kb0, int nkb,
                                               int lane)
{
    int it = 0;
    for (; it + 3 <= nkb; it += 3) {
        wave_block<kChain, kFmtA, kFmtB>(p, s, s0, s2, acc, o, w, kb0 + it + 2, it + 2 < nkb, lane);
        wave_block<kChain, kFmtA, kFmtB>(p, s, s1, s0, acc, o, w, kb0 + it + 3, it + 3 < nkb, lane);
        wave_block<kChain, kFmtA, kFmtB>(p, s, s2, s1, acc, o, w, kb0 + it + 4, it + 4 < nkb, lane);
    }
    if (it < nkb) wave_block<kChain, kFmtA, kFmtB>(p, s, s0, s2, acc, o, w, kb0 + it + 2, it + 2 < nkb, lane);
    if (it + 1 < nkb) wave_block<kChain, kFmtA, kFmtB>(p, s, s1, s0, acc, o, w, kb0 + it + 3, it + 3 < nkb, lane);
    // the trailing copies (empty ranges) still write LDS: let them land
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int kFmtA, int kFmtB, bool kFast, int kEpi, int kQuant>
__global__ __launch_bounds__(kVThreads) void gemm_nt_wave_kernel(const GemmArgs p)
{
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kVStages * kVStage];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wave = (int)(blockIdx.x % kWaves);          // the wave tile's place in its 256 x 256 tile
    const TileCtx c = tile_ctx(p, (int64_t)(blockIdx.x / kWaves));
    const int wm = wave / kWavesN, wn = wave % kWavesN;
    const int64_t m0 = c.m0 + wm * kWM, n0 = c.n0 + wn * kWN;
    // (an empty group's or a skipped block's tile leaves its output untouched)
    if (n0 >= p.N || c.nkb == 0) return;
    if (m0 >= p.M) {
        // no rows: only the deterministic bias gradient's workspace row of this
        // wave place is due (zero, as the persistent kernel's wave writes it)
        if (w == 0 && kEpi == (int)Epi::Dgrad && (p.flags & TE_EPI_BGRAD) && p.bgrad_ws) {
            float* row = p.bgrad_ws + ((c.m0 / kBM) * kWavesM + wm) * p.bgrad_ws_ld;
            for (int n = lane; n < kWN; n += 64)
                if (n0 + n < p.N) row[n0 + n] = 0.0f;
        }
        return;
    }
    WaveSrc s;
    s.a = make_rsrc(p.a + m0 * p.lda, min((int64_t)kWM, p.M - m0) * p.lda);
    s.b = make_rsrc(p.b + c.bgrp * p.b_group_stride + n0 * p.ldb, min((int64_t)kWN, p.N - n0) * p.ldb);
    s.sa = p.sa + m0;
    s.sb = p.sb + c.bgrp * p.sb_group_stride + n0;
    s.sa_bytes = (int)(min((int64_t)kWM, p.lsa - m0) * 4);
    s.sb_bytes = (int)(min((int64_t)kWN, p.lsb - n0) * 4);
    const int kb0 = c.kb0, nkb = c.nkb;
    const bool chain = kFast && wave_scales_pow2(p, s, m0, n0, kb0, nkb, lane);

    WaveLane o;
    o.r16 = lane & 15;
    o.q4 = lane >> 4;
    o.a_lo = swz(o.r16, o.q4);
    o.a_hi = swz(o.r16, o.q4 + 4);
    o.b_lo = kVA + swz(o.r16, o.q4);
    o.b_hi = kVA + swz(o.r16, o.q4 + 4);
    // (stage offsets hidden from the compiler: folded to constants they lose
    // the restrict scopes the loop's waits rely on)
    int s0_off = 0, s1_off = kVStage, s2_off = 2 * kVStage;
    asm volatile("" : "+s"(s0_off), "+s"(s1_off), "+s"(s2_off));
    wave_load_part(p, s, smem, kb0, 0 < nkb, w, lane);
    wave_load_part(p, s, smem + kVStage, kb0 + 1, 1 < nkb, w, lane);

    v4f part[kTM][kVJ];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int jj = 0; jj < kVJ; ++jj) part[i][jj] = v4f{0.f, 0.f, 0.f, 0.f};
    if (chain)
        wave_main_loop<true, kFmtA, kFmtB>(p, s, smem + s0_off, smem + s1_off, smem + s2_off, part, o, w, kb0, nkb,
                                           lane);
    else
        wave_main_loop<false, kFmtA, kFmtB>(p, s, smem + s0_off, smem + s1_off, smem + s2_off, part, o, w, kb0, nkb,
                                            lane);

    const uint16_t* bias_v = p.bias + c.bgrp * p.bias_group_stride;
    float* bgrad_v = p.bias_grad + c.bgrp * p.bias_group_stride;
    if constexpr (kQuant == 0) {
        // wave w's share: columns 32 w .. 32 w + 31 of the wave tile
        const int64_t nw = c.n0 + w * (kVJ * 16);
        if (m0 + kWM <= p.M && n0 + (w + 1) * (kVJ * 16) <= p.N)
            epilogue<kEpi, true, 0, kVJ>(p, part, c.m0, nw, c.out_off, bias_v, bgrad_v, smem, wave, lane);
        else
            epilogue<kEpi, false, 0, kVJ>(p, part, c.m0, nw, c.out_off, bias_v, bgrad_v, smem, wave, lane);
        return;
    }
    // the four waves' column groups meet in wave 0 (value r of wave w at
    // [(w * 32 + r) * 64 + lane]: one dword per lane, no bank conflicts)
    float* G = reinterpret_cast<float*>(smem);
    __syncthreads();   // every wave is done reading the stages
    if (w != 0) {
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int jj = 0; jj < kVJ; ++jj)
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) G[(w * 32 + (i * kVJ + jj) * 4 + cc) * 64 + lane] = part[i][jj][cc];
    }
    __syncthreads();
    if (w != 0) return;
    v4f acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            const int ww = j / kVJ, jj = j % kVJ;
            if (ww == 0) {
                acc[i][j] = part[i][jj];
            } else {
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) acc[i][j][cc] = G[(ww * 32 + (i * kVJ + jj) * 4 + cc) * 64 + lane];
            }
        }
    epilogue<kEpi, false, kQuant>(p, acc, c.m0, c.n0, c.out_off, bias_v, bgrad_v, smem, wave, lane);
}

#if TE_GEMM_PART < 0 || TE_GEMM_PART == 4
__global__ void zero_f32_kernel(float* p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// The second pass of the deterministic bias gradient: one thread per column
// sums the workspace rows in order (coalesced across the threads of a row).
constexpr int kReduceThreads = 64;  // one column per thread; small workgroups spread the columns over the CUs
constexpr int kReduceChunk = 32;    // rows whose loads are in flight together

__global__ __launch_bounds__(kReduceThreads) void bgrad_reduce_kernel(const float* __restrict__ ws, int64_t rows,
                                                                      int64_t ld, int64_t N,
                                                                      float* __restrict__ bias_grad)
{
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    // The rows are summed in order; their loads go out kReduceChunk at a time
    // (one load after another cost a memory round trip per row: 44.6 us for
    // the 128 rows x 14336 columns of an 8192 x 14336 bias gradient).
    float s = 0.0f;
    for (int64_t r0 = 0; r0 < rows; r0 += kReduceChunk) {
        float v[kReduceChunk];
#pragma unroll
        for (int u = 0; u < kReduceChunk; ++u) v[u] = r0 + u < rows ? ws[(r0 + u) * ld + n] : 0.0f;
#pragma unroll
        for (int u = 0; u < kReduceChunk; ++u)
            if (r0 + u < rows) s += v[u];
    }
    bias_grad[n] = s;
}

// The M-grouped form: bias_grad[e][n] sums, in block order, the four
// workspace rows of every 256-row block whose expert is e (a skipped block's
// rows were never written and are not read; an expert with no block gets 0).
__global__ void mgrouped_bgrad_reduce_kernel(const float* __restrict__ ws, int64_t blocks, int64_t ld, int64_t N,
                                             int32_t G, const int32_t* __restrict__ m_block_group,
                                             float* __restrict__ bias_grad)
{
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int32_t e = (int32_t)blockIdx.y;
    if (n >= N || e >= G) return;
    float s = 0.0f;
    for (int64_t b = 0; b < blocks; ++b) {
        if (m_block_group[b] != e) continue;
#pragma unroll
        for (int r = 0; r < kBgradRowsPerTile; ++r) s += ws[(b * kBgradRowsPerTile + r) * ld + n];
    }
    bias_grad[(int64_t)e * N + n] = s;
}

#endif

template <int kFmtA, int kFmtB, bool kFast>
hipError_t launch_epi(const GemmArgs& a, dim3 grid, int64_t tiles, hipStream_t s)
{
    // (the quantising stores are kernels of their own: their registers stay out
    // of the plain epilogues, and the transposed store's, which holds the whole
    // tile until its column maxima are known, out of the row-wise one)
    const int qz = a.qt_out != nullptr ? 2 : (a.q_out != nullptr ? 1 : 0);
    switch (a.epi) {
    case Epi::Wgrad: gemm_nt_kernel<kFmtA, kFmtB, kFast, (int)Epi::Wgrad, 0><<<grid, kThreads, 0, s>>>(a, tiles); break;
    case Epi::Fwd:
        if (qz == 2) gemm_nt_kernel<kFmtA, kFmtB, kFast, (int)Epi::Fwd, 2><<<grid, kThreads, 0, s>>>(a, tiles);
        else if (qz == 1) gemm_nt_kernel<kFmtA, kFmtB, kFast, (int)Epi::Fwd, 1><<<grid, kThreads, 0, s>>>(a, tiles);
        else gemm_nt_kernel<kFmtA, kFmtB, kFast, (int)Epi::Fwd, 0><<<grid, kThreads, 0, s>>>(a, tiles);
        break;
    case Epi::Dgrad:
        if (qz == 2) gemm_nt_kernel<kFmtA, kFmtB, kFast, (int)Epi::Dgrad, 2><<<grid, kThreads, 0, s>>>(a, tiles);
        else if (qz == 1) gemm_nt_kernel<kFmtA, kFmtB, kFast, (int)Epi::Dgrad, 1><<<grid, kThreads, 0, s>>>(a, tiles);
        else gemm_nt_kernel<kFmtA, kFmtB, kFast, (int)Epi::Dgrad, 0><<<grid, kThreads, 0, s>>>(a, tiles);
        break;
    }
    return hipGetLastError();
}

// (every product but the transposed quantising store: launch_gemm's choice)
template <int kFmtA, int kFmtB, bool kFast>
hipError_t launch_wave_epi(const GemmArgs& a, dim3 grid, hipStream_t s)
{
    const bool q = a.q_out != nullptr;
    switch (a.epi) {
    case Epi::Wgrad: gemm_nt_wave_kernel<kFmtA, kFmtB, kFast, (int)Epi::Wgrad, 0><<<grid, kVThreads, 0, s>>>(a); break;
    case Epi::Fwd:
        if (q) gemm_nt_wave_kernel<kFmtA, kFmtB, kFast, (int)Epi::Fwd, 1><<<grid, kVThreads, 0, s>>>(a);
        else gemm_nt_wave_kernel<kFmtA, kFmtB, kFast, (int)Epi::Fwd, 0><<<grid, kVThreads, 0, s>>>(a);
        break;
    case Epi::Dgrad:
        if (q) gemm_nt_wave_kernel<kFmtA, kFmtB, kFast, (int)Epi::Dgrad, 1><<<grid, kVThreads, 0, s>>>(a);
        else gemm_nt_wave_kernel<kFmtA, kFmtB, kFast, (int)Epi::Dgrad, 0><<<grid, kVThreads, 0, s>>>(a);
        break;
    }
    return hipGetLastError();
}

template <int kFmtA, int kFmtB>
hipError_t launch_policy(const GemmArgs& a, dim3 grid, int64_t tiles, hipStream_t s)
{
    return a.fast ? launch_epi<kFmtA, kFmtB, true>(a, grid, tiles, s)
                  : launch_epi<kFmtA, kFmtB, false>(a, grid, tiles, s);
}

template <int kFmtA, int kFmtB>
hipError_t launch_wave_policy(const GemmArgs& a, dim3 grid, hipStream_t s)
{
    return a.fast ? launch_wave_epi<kFmtA, kFmtB, true>(a, grid, s) : launch_wave_epi<kFmtA, kFmtB, false>(a, grid, s);
}

}  // namespace

// One translation unit per operand-format pair for the persistent kernels
// (TE_GEMM_PART 0-3), one per pair for the wave kernels (5-8: in a unit of
// their own, the persistent kernels' register allocation stays as it is) and
// one for the host side (4), so the instantiations compile in parallel;
// without TE_GEMM_PART everything is in one unit.
hipError_t launch_pair_e4_e4(const GemmArgs& a, dim3 grid, int64_t tiles, hipStream_t s);
hipError_t launch_wave_pair_e4_e4(const GemmArgs& a, dim3 grid, hipStream_t s);
hipError_t launch_pair_e5_e4(const GemmArgs& a, dim3 grid, int64_t tiles, hipStream_t s);
hipError_t launch_wave_pair_e5_e4(const GemmArgs& a, dim3 grid, hipStream_t s);
hipError_t launch_pair_e4_e5(const GemmArgs& a, dim3 grid, int64_t tiles, hipStream_t s);
hipError_t launch_wave_pair_e4_e5(const GemmArgs& a, dim3 grid, hipStream_t s);
hipError_t launch_pair_e5_e5(const GemmArgs& a, dim3 grid, int64_t tiles, hipStream_t s);
hipError_t launch_wave_pair_e5_e5(const GemmArgs& a, dim3 grid, hipStream_t s);
#if TE_GEMM_PART < 0 || TE_GEMM_PART == 0
hipError_t launch_pair_e4_e4(const GemmArgs& a, dim3 grid, int64_t tiles, hipStream_t s)
{
    return launch_policy<FMT_E4M3, FMT_E4M3>(a, grid, tiles, s);
}
#endif
#if TE_GEMM_PART < 0 || TE_GEMM_PART == 5
hipError_t launch_wave_pair_e4_e4(const GemmArgs& a, dim3 grid, hipStream_t s)
{
    return launch_wave_policy<FMT_E4M3, FMT_E4M3>(a, grid, s);
}
#endif
#if TE_GEMM_PART < 0 || TE_GEMM_PART == 1
hipError_t launch_pair_e5_e4(const GemmArgs& a, dim3 grid, int64_t tiles, hipStream_t s)
{
    return launch_policy<FMT_E5M2, FMT_E4M3>(a, grid, tiles, s);
}
#endif
#if TE_GEMM_PART < 0 || TE_GEMM_PART == 6
hipError_t launch_wave_pair_e5_e4(const GemmArgs& a, dim3 grid, hipStream_t s)
{
    return launch_wave_policy<FMT_E5M2, FMT_E4M3>(a, grid, s);
}
#endif
#if TE_GEMM_PART < 0 || TE_GEMM_PART == 2
hipError_t launch_pair_e4_e5(const GemmArgs& a, dim3 grid, int64_t tiles, hipStream_t s)
{
    return launch_policy<FMT_E4M3, FMT_E5M2>(a, grid, tiles, s);
}
#endif
#if TE_GEMM_PART < 0 || TE_GEMM_PART == 7
hipError_t launch_wave_pair_e4_e5(const GemmArgs& a, dim3 grid, hipStream_t s)
{
    return launch_wave_policy<FMT_E4M3, FMT_E5M2>(a, grid, s);
}
#endif
#if TE_GEMM_PART < 0 || TE_GEMM_PART == 3
hipError_t launch_pair_e5_e5(const GemmArgs& a, dim3 grid, int64_t tiles, hipStream_t s)
{
    return launch_policy<FMT_E5M2, FMT_E5M2>(a, grid, tiles, s);
}
#endif
#if TE_GEMM_PART < 0 || TE_GEMM_PART == 8
hipError_t launch_wave_pair_e5_e5(const GemmArgs& a, dim3 grid, hipStream_t s)
{
    return launch_wave_policy<FMT_E5M2, FMT_E5M2>(a, grid, s);
}
#endif

#if TE_GEMM_PART < 0 || TE_GEMM_PART == 4
// Compute units of the current device (cached per device).
int device_cus()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Which kernel takes a product: the wave-tile one when the 256 x 256 tiles
// (of all groups together) number at most a quarter of the compute units (its
// workgroups, one per wave tile, then fill every CU at most twice over), the
// persistent one otherwise.  Kernel trace, out += A B^T (FULL), wave against
// persistent: 1 and 4 tiles, K = 512: 8.7-8.8 vs 21.2-21.5 us; K = 2048:
// 16.2 vs 36.6 us; 32 tiles (1024 x 2048), K = 4096: 29.8 vs 60.1 us; 64
// tiles (2048 x 2048): 39.2 vs 61.9 us; 128 tiles (2048 x 4096): 33.3 vs 33.2
// us at K = 1024 but 72.1 vs 64.5 us at K = 4096, where the persistent
// kernel's eight waves per tile are ahead.  The environment variable
// TE_FP8_GEMM_PATH ("wave" or "persistent") overrides the choice for the
// products the wave kernel supports.
bool use_wave_path(const GemmArgs& a, int64_t tiles, int cus)
{
    const bool supported = !a.qt_out;
    if (!supported) return false;
    const char* env = std::getenv("TE_FP8_GEMM_PATH");
    if (env && std::strcmp(env, "wave") == 0) return true;
    if (env && std::strcmp(env, "persistent") == 0) return false;
    return tiles * 4 <= cus;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream, LaunchInfo* info)
{
    const int64_t tiles = ((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN) * a.num_groups;
    const int cus = device_cus();
    const bool wave_path = use_wave_path(a, tiles, cus);
    // persistent: one workgroup per compute unit (the two stages fill most of its
    // LDS); wave path: one four-wave workgroup per wave tile
    const int64_t blocks = wave_path ? tiles * kWaves : std::min<int64_t>(tiles, cus);
    if (info) {
        info->tile_m = wave_path ? kWM : kBM;
        info->tile_n = wave_path ? kWN : kBN;
        info->threads = wave_path ? kVThreads : kThreads;
        info->grid = blocks;
    }
    if (blocks <= 0) return hipSuccess;
    const dim3 grid((unsigned)blocks);
    if (wave_path) {
        if (a.fmt_a == FMT_E4M3 && a.fmt_b == FMT_E4M3) return launch_wave_pair_e4_e4(a, grid, stream);
        if (a.fmt_a == FMT_E5M2 && a.fmt_b == FMT_E4M3) return launch_wave_pair_e5_e4(a, grid, stream);
        if (a.fmt_a == FMT_E4M3 && a.fmt_b == FMT_E5M2) return launch_wave_pair_e4_e5(a, grid, stream);
        return launch_wave_pair_e5_e5(a, grid, stream);
    }
    if (a.fmt_a == FMT_E4M3 && a.fmt_b == FMT_E4M3) return launch_pair_e4_e4(a, grid, tiles, stream);
    if (a.fmt_a == FMT_E5M2 && a.fmt_b == FMT_E4M3) return launch_pair_e5_e4(a, grid, tiles, stream);
    if (a.fmt_a == FMT_E4M3 && a.fmt_b == FMT_E5M2) return launch_pair_e4_e5(a, grid, tiles, stream);
    return launch_pair_e5_e5(a, grid, tiles, stream);
}

// Scratch of the entry point that allocates nothing: the column-sum
// workspace of the deterministic bias gradient.  Each GPU holds its own copy
// for the life of the process.  In host code `scratch` names a host-side
// stand-in, never the device memory: only the address returned by
// hipGetSymbolAddress on the device in question may reach a kernel or a copy.
static __device__ __align__(256) float scratch[TE_NOALLOC_SCRATCH_BYTES / sizeof(float)];

hipError_t noalloc_scratch(void** ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with device `dev` current
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_bgrad_reduce(const float* ws, int64_t rows, int64_t ld, int64_t N, float* bias_grad,
                               hipStream_t stream)
{
    if (N <= 0) return hipSuccess;
    bgrad_reduce_kernel<<<(unsigned)((N + kReduceThreads - 1) / kReduceThreads), kReduceThreads, 0, stream>>>(
        ws, rows, ld, N, bias_grad);
    return hipGetLastError();
}

hipError_t launch_mgrouped_bgrad_reduce(const float* ws, int64_t blocks, int64_t ld, int64_t N, int32_t G,
                                        const int32_t* m_block_group, float* bias_grad, hipStream_t stream)
{
    if (N <= 0 || G <= 0) return hipSuccess;
    const dim3 grid((unsigned)((N + 255) / 256), (unsigned)G);
    mgrouped_bgrad_reduce_kernel<<<grid, 256, 0, stream>>>(ws, blocks, ld, N, G, m_block_group, bias_grad);
    return hipGetLastError();
}

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    zero_f32_kernel<<<(unsigned)blocks, 256, 0, stream>>>(p, n);
    return hipGetLastError();
}
#endif

}  // namespace tefp8
