// Per-token 1x128 fp8 cast for gfx950.
//
// For every row and every 128-column group: amax over the group, a fp32
// dequantisation scale s = amax_c / FP8_MAX (or the power of two just above
// it), and codes q = RNE_sat(x * FP8_MAX / amax_c).  The step is named (not
// defined) by the worked example on "Weight gradient kernels for dense and MoE
// models" (DeepGEMM pull request 95), which casts both wgrad operands per
// token before the GEMM; the 128-wide groups and the reading of s are this
// library's definition (see te_fp8.h).
//
// Scales are written block-major, scales[group * ld_s + row], so that the GEMM
// reads the scales of one 128-deep block as one contiguous vector.
//
// Memory-bound: 2 bytes read and 1 byte + 1/32 byte written per element.  One
// group is handled by 8 consecutive lanes, 16 elements each: lane p of the
// group takes elements 8p .. 8p + 7 and 64 + 8p .. 64 + 8p + 7, so each of its
// two 16-byte loads is, across the 8 lanes, one whole 128-byte line of the
// row (with 16 contiguous elements per lane instead, every load instruction
// touched twice the lines, each half used: 6-9 % slower).  A workgroup covers
// a tile of 32 rows x 2 groups (256 columns; 4 and 8 groups per tile were
// slower, 1 no faster): each wave takes 8 rows, each lane the same slices of
// its row in the 2 groups, so a thread has its 4 16-byte loads in flight
// together, and the 32 rows' scales of a group (adjacent in the block-major
// layout) are one 128-byte line written by one workgroup.
// The group max is a 3-step DPP butterfly inside the 8 lanes.  The fp32 -> fp8
// rounding is the hardware v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 on inputs
// clamped to +-FP8_MAX (round to nearest even; the clamp gives saturation).
//
// The fused cast-transpose reads each 128 x 128 bf16 tile once (persistent
// workgroups, the next tile's loads in flight during the current one).  The row-wise
// cast works from the loaded registers (16 lanes per row, 8 elements each,
// a 4-step DPP max over the 16 lanes); the tile also goes to LDS, from which
// 8 lanes per column read 16 consecutive rows each for the cast of the
// transpose.  Chunk c (16 bytes) of LDS row r sits at slot c ^ ((r >> 4) & 15),
// so the 2-byte column reads of a wave (8 columns x 8 row segments 16 rows
// apart) fall in distinct banks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "fp8_codec.h"
#include "internal.h"

namespace tefp8 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kLanesPerGroup = 8;

// DPP controls (row_* act within 16-lane rows).
constexpr int kQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7-i within each half row

template <int kCtrl>
__device__ __forceinline__ float max_with_dpp(float v)
{
    int o = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false);
    return fmaxf(v, __builtin_bit_cast(float, o));
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

constexpr int kTileRows = 32;   // 4 waves x 8 rows
constexpr int kTileGroups = 2;  // 128-column groups per tile

// One 32-row x 256-column tile of one operand.
template <int kFmt, bool kPow2>
__device__ __forceinline__ void cast_tile(const CastOperand& o, int64_t tile)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int part = lane & (kLanesPerGroup - 1);
    const int64_t tile_r = tile / o.tiles_c;
    const int64_t tile_c = tile - tile_r * o.tiles_c;
    const int64_t row_raw = tile_r * kTileRows + wave * 8 + (lane >> 3);
    // Rows and groups past the end repeat the last valid one (the 8 lanes of
    // a group stay together, so the DPP exchange is unaffected) and store
    // nothing.
    const bool row_ok = row_raw < o.rows;
    const int64_t row = row_ok ? row_raw : o.rows - 1;
    const int64_t g0 = tile_c * kTileGroups;

    u32x4 u[kTileGroups][2];
#pragma unroll
    for (int t = 0; t < kTileGroups; ++t) {
        const int64_t gc = min(g0 + t, o.gpr - 1);
        const uint16_t* src = o.x + row * o.ld_x + gc * 128 + part * 8;
        u[t][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
        u[t][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + 64));
    }
#pragma unroll
    for (int t = 0; t < kTileGroups; ++t) {
        const uint32_t w[8] = {u[t][0][0], u[t][0][1], u[t][0][2], u[t][0][3],
                               u[t][1][0], u[t][1][1], u[t][1][2], u[t][1][3]};
        float v[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = bf16lo(w[i]);
            v[2 * i + 1] = bf16hi(w[i]);
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
        amax = max_with_dpp<kQuadXor1>(amax);
        amax = max_with_dpp<kQuadXor2>(amax);
        amax = max_with_dpp<kRowHalfMirror>(amax);

        float scale, mult;
        group_scale<kFmt, kPow2>(amax, scale, mult);
        float s0[8], s1[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            s0[i] = v[i] * mult;
            s1[i] = v[8 + i] * mult;
        }
        const uint2 c0 = encode8<kFmt>(s0);
        const uint2 c1 = encode8<kFmt>(s1);
        const int64_t gc = g0 + t;
        if (row_ok && gc < o.gpr) {
            *reinterpret_cast<uint2*>(o.q + row * o.ld_q + gc * 128 + part * 8) = c0;
            *reinterpret_cast<uint2*>(o.q + row * o.ld_q + gc * 128 + 64 + part * 8) = c1;
            if (part == 0) o.scales[gc * o.ld_s + row] = scale;  // block-major: [cols/128][ld_s]
        }
    }
}

// One launch over the tiles of up to kMaxCastBatch operands: workgroup w
// casts tile w - tile_begin of the last operand whose tiles begin at or
// before w.
template <int kFmt, bool kPow2>
__global__ __launch_bounds__(kThreads) void cast_per_token_kernel(const CastBatch b)
{
    const int64_t w = blockIdx.x;
    int k = 0;
    for (int i = 1; i < b.n; ++i)
        if (w >= b.op[i].tile_begin) k = i;
    const CastOperand* ops = b.op;
    cast_tile<kFmt, kPow2>(ops[k], w - ops[k].tile_begin);
}

// ------------------------------------------------------------ cast-transpose
constexpr int kCT = 128;              // tile side (one group in each direction)
constexpr int kRowMirror = 0x140;      // lane i <-> 15-i within each 16-lane row

// Load one 128 x 128 tile: 2048 chunks of 8 bf16, chunk u * 256 + t is row
// 16 u + (t >> 4), chunk t & 15 of that row.  Columns past `cols` (only in the
// last tile column, without the row-wise cast) read as zero.
__device__ __forceinline__ void load_tile(u32x4 (&v)[8], const uint16_t* __restrict__ x, int64_t cols,
                                          int64_t tiles_c, int64_t ld_x, int64_t tile)
{
    const int t = threadIdx.x, cc = t & 15;
    const int64_t tr = tile / tiles_c;
    const int64_t r0 = tr * kCT, c0 = (tile - tr * tiles_c) * kCT;
    const bool chunk_in = c0 + cc * 8 < cols;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int r = 16 * u + (t >> 4);
        v[u] = u32x4{0u, 0u, 0u, 0u};
        if (chunk_in)
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + (r0 + r) * ld_x + c0 + cc * 8));
    }
}

// Persistent: workgroup w casts tiles w, w + G, ...; the next tile's loads are
// in flight while the current one is cast.
template <int kFmt, bool kPow2, bool kRowwise>
__global__ __launch_bounds__(kThreads) void cast_transpose_kernel(
    const uint16_t* __restrict__ x, int64_t cols, int64_t tiles_c, int64_t total_tiles, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scales, int64_t ld_s, uint8_t* __restrict__ qt,
    int64_t ld_qt, float* __restrict__ scales_t, int64_t ld_st)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[kCT * kCT * 2];
    const int t = threadIdx.x;
    const int cc = t & 15;

    int64_t id = blockIdx.x;
    u32x4 v[8];
    load_tile(v, x, cols, tiles_c, ld_x, id);
    for (; id < total_tiles; id += gridDim.x) {
        const int64_t tr = id / tiles_c;
        const int64_t r0 = tr * kCT, c0 = (id - tr * tiles_c) * kCT;
        const int64_t next = id + gridDim.x;
        u32x4 vn[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) vn[u] = u32x4{0u, 0u, 0u, 0u};
        if (next < total_tiles) load_tile(vn, x, cols, tiles_c, ld_x, next);

#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int r = 16 * u + (t >> 4);
            *reinterpret_cast<u32x4*>(tile + r * (kCT * 2) + ((cc ^ ((r >> 4) & 15)) << 4)) = v[u];
        }

        if (kRowwise) {
            // row-wise groups: the 16 lanes of a DPP row hold one row's 128 columns
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int r = 16 * u + (t >> 4);
                float f[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f[2 * i] = bf16lo(v[u][i]);
                    f[2 * i + 1] = bf16hi(v[u][i]);
                }
                float amax = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
                amax = max_with_dpp<kQuadXor1>(amax);
                amax = max_with_dpp<kQuadXor2>(amax);
                amax = max_with_dpp<kRowHalfMirror>(amax);
                amax = max_with_dpp<kRowMirror>(amax);
                float scale, mult;
                group_scale<kFmt, kPow2>(amax, scale, mult);
#pragma unroll
                for (int i = 0; i < 8; ++i) f[i] *= mult;
                const uint2 c = encode8<kFmt>(f);
                *reinterpret_cast<uint2*>(q + (r0 + r) * ld_q + c0 + cc * 8) = c;
                if (cc == 0) scales[(c0 / kCT) * ld_s + r0 + r] = scale;
            }
        }
        __syncthreads();

        // transposed groups: 8 lanes per column, lane `part` takes rows 16 part .. 16 part + 15
        const int part = t & 7;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int col = 32 * u + (t >> 3);
            float f[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int r = 16 * part + k;
                const uint16_t h = *reinterpret_cast<const uint16_t*>(
                    tile + r * (kCT * 2) + (((col >> 3) ^ ((r >> 4) & 15)) << 4) + (col & 7) * 2);
                f[k] = __builtin_bit_cast(float, (uint32_t)h << 16);
            }
            float amax = 0.0f;
#pragma unroll
            for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fabsf(f[k]));
            amax = max_with_dpp<kQuadXor1>(amax);
            amax = max_with_dpp<kQuadXor2>(amax);
            amax = max_with_dpp<kRowHalfMirror>(amax);
            float scale, mult;
            group_scale<kFmt, kPow2>(amax, scale, mult);
            float s0[8], s1[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                s0[i] = f[i] * mult;
                s1[i] = f[8 + i] * mult;
            }
            const uint2 e0 = encode8<kFmt>(s0);
            const uint2 e1 = encode8<kFmt>(s1);
            if (c0 + col < cols) {
                *reinterpret_cast<uint4*>(qt + (c0 + col) * ld_qt + r0 + part * 16) = make_uint4(e0.x, e0.y, e1.x, e1.y);
                if (part == 0) scales_t[(r0 / kCT) * ld_st + c0 + col] = scale;
            }
        }
        __syncthreads();  // the tile buffer is rewritten by the next iteration
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = vn[u];
    }
}

// ------------------------------------------------------------ operand row sums
// bias_grad[r] = sum_k dec(q[r][k]) * s(r, k/128): one wave per row, lane l
// decodes 16 consecutive codes of each 1 KiB chunk (8 lanes per 128-element
// scale block), multiplies its partial sum by that block's scale, and the
// wave sums its lanes at the end.
// The fp8 code in byte kB of w as fp32 (exact).
template <int kFmt, int kB>
__device__ __forceinline__ float dec_byte(uint32_t w)
{
    if (kFmt == FMT_E4M3) return __builtin_amdgcn_cvt_f32_fp8((int)w, kB);
    return __builtin_amdgcn_cvt_f32_bf8((int)w, kB);
}

template <int kFmt>
__global__ __launch_bounds__(kThreads) void row_sum_kernel(const uint8_t* __restrict__ q, int64_t rows, int64_t cols,
                                                          int64_t ld_q, const float* __restrict__ scales,
                                                          int64_t ld_s, float* __restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (r >= rows) return;   // whole waves only: r is uniform in a wave
    float acc = 0.0f;
    for (int64_t c0 = 0; c0 < cols; c0 += 1024) {
        const int64_t c = c0 + lane * 16;
        if (c < cols) {
            const uint4 w = *reinterpret_cast<const uint4*>(q + r * ld_q + c);
            const uint32_t d[4] = {w.x, w.y, w.z, w.w};
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                part += (dec_byte<kFmt, 0>(d[i]) + dec_byte<kFmt, 1>(d[i])) +
                        (dec_byte<kFmt, 2>(d[i]) + dec_byte<kFmt, 3>(d[i]));
            acc = fmaf(part, scales[(c / 128) * ld_s + r], acc);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) out[r] = acc;
}

}  // namespace

hipError_t launch_cast_batch(const CastOperand* ops, int n, int fmt, bool pow2, hipStream_t stream, LaunchInfo* info)
{
    if (n < 1 || n > kMaxCastBatch) return hipErrorInvalidValue;
    CastBatch b{};
    b.n = n;
    int64_t blocks = 0;
    for (int i = 0; i < n; ++i) {
        b.op[i] = ops[i];
        b.op[i].gpr = ops[i].cols / 128;
        b.op[i].tiles_c = (b.op[i].gpr + kTileGroups - 1) / kTileGroups;
        b.op[i].tile_begin = blocks;
        blocks += ((ops[i].rows + kTileRows - 1) / kTileRows) * b.op[i].tiles_c;
    }
    if (info) { info->tile_m = kTileRows; info->tile_n = 128 * kTileGroups; info->threads = kThreads; info->grid = blocks; }
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (blocks <= 0) return hipSuccess;
    dim3 grid((unsigned)blocks), block(kThreads);
    if (fmt == FMT_E4M3) {
        if (pow2) cast_per_token_kernel<FMT_E4M3, true><<<grid, block, 0, stream>>>(b);
        else cast_per_token_kernel<FMT_E4M3, false><<<grid, block, 0, stream>>>(b);
    } else {
        if (pow2) cast_per_token_kernel<FMT_E5M2, true><<<grid, block, 0, stream>>>(b);
        else cast_per_token_kernel<FMT_E5M2, false><<<grid, block, 0, stream>>>(b);
    }
    return hipGetLastError();
}

hipError_t launch_row_sum(const uint8_t* q, int64_t rows, int64_t cols, int64_t ld_q, int fmt, const float* scales,
                          int64_t ld_s, float* out, hipStream_t stream)
{
    const int64_t blocks = (rows + kThreads / 64 - 1) / (kThreads / 64);
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (fmt == FMT_E4M3)
        row_sum_kernel<FMT_E4M3><<<(unsigned)blocks, kThreads, 0, stream>>>(q, rows, cols, ld_q, scales, ld_s, out);
    else
        row_sum_kernel<FMT_E5M2><<<(unsigned)blocks, kThreads, 0, stream>>>(q, rows, cols, ld_q, scales, ld_s, out);
    return hipGetLastError();
}

hipError_t launch_cast(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int fmt,
                       bool pow2, uint8_t* q, int64_t ld_q, float* scales, int64_t ld_s, hipStream_t stream,
                       LaunchInfo* info)
{
    CastOperand o{};
    o.x = x;
    o.rows = rows;
    o.cols = cols;
    o.ld_x = ld_x;
    o.q = q;
    o.ld_q = ld_q;
    o.scales = scales;
    o.ld_s = ld_s;
    return launch_cast_batch(&o, 1, fmt, pow2, stream, info);
}

hipError_t launch_cast_transpose(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int fmt, bool pow2,
                                 uint8_t* q, int64_t ld_q, float* scales, int64_t ld_s, uint8_t* qt, int64_t ld_qt,
                                 float* scales_t, int64_t ld_st, hipStream_t stream, LaunchInfo* info)
{
    const int64_t tiles_c = (cols + kCT - 1) / kCT;
    const int64_t tiles = (rows / kCT) * tiles_c;
    // four resident workgroups per compute unit (32 KiB of LDS each)
    const int64_t blocks = std::min<int64_t>(tiles, 4 * (int64_t)device_cus());
    if (info) { info->tile_m = kCT; info->tile_n = kCT; info->threads = kThreads; info->grid = blocks; }
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (blocks <= 0) return hipSuccess;
    const dim3 grid((unsigned)blocks), block(kThreads);
#define TE_CT_LAUNCH(F, P, R) \
    cast_transpose_kernel<F, P, R><<<grid, block, 0, stream>>>(x, cols, tiles_c, tiles, ld_x, q, ld_q, scales, ld_s, qt, ld_qt, scales_t, ld_st)
    const bool rw = q != nullptr;
    if (fmt == FMT_E4M3) {
        if (pow2) { if (rw) TE_CT_LAUNCH(FMT_E4M3, true, true); else TE_CT_LAUNCH(FMT_E4M3, true, false); }
        else { if (rw) TE_CT_LAUNCH(FMT_E4M3, false, true); else TE_CT_LAUNCH(FMT_E4M3, false, false); }
    } else {
        if (pow2) { if (rw) TE_CT_LAUNCH(FMT_E5M2, true, true); else TE_CT_LAUNCH(FMT_E5M2, true, false); }
        else { if (rw) TE_CT_LAUNCH(FMT_E5M2, false, true); else TE_CT_LAUNCH(FMT_E5M2, false, false); }
    }
#undef TE_CT_LAUNCH
    return hipGetLastError();
}

}  // namespace tefp8
