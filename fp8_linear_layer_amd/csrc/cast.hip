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
// group is handled by 8 consecutive lanes, 16 elements (32 bytes) each.  A
// workgroup covers a tile of 32 rows x 4 groups (512 columns): each wave takes
// 8 rows, each lane the same 16-element slice of its row in the 4 groups, so
// a thread has its 8 16-byte loads in flight together, a row's 1 KiB of input
// is read by 8 lanes as one run, and the 32 rows' scales of a group (adjacent
// in the block-major layout) are one 128-byte line written by one workgroup.
// The group max is a 3-step DPP butterfly inside the 8 lanes.  The fp32 -> fp8
// rounding is the hardware v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 on inputs
// clamped to +-FP8_MAX (round to nearest even; the clamp gives saturation).
#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Eight fp32 values (already scaled) -> eight fp8 codes in two dwords.
template <int kFmt>
__device__ __forceinline__ uint2 encode8(const float (&v)[8], float fmax)
{
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float a = __builtin_amdgcn_fmed3f(v[4 * h + 0], -fmax, fmax);
        float b = __builtin_amdgcn_fmed3f(v[4 * h + 1], -fmax, fmax);
        float c = __builtin_amdgcn_fmed3f(v[4 * h + 2], -fmax, fmax);
        float d = __builtin_amdgcn_fmed3f(v[4 * h + 3], -fmax, fmax);
        int p;
        if (kFmt == FMT_E4M3) {
            p = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
            p = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, p, true);
        } else {
            p = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
            p = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, p, true);
        }
        w[h] = (uint32_t)p;
    }
    return make_uint2(w[0], w[1]);
}

constexpr int kTileRows = 32;   // 4 waves x 8 rows
constexpr int kTileGroups = 4;  // 128-column groups per tile

template <int kFmt, bool kPow2>
__device__ __forceinline__ void group_scale(float amax, float& scale, float& mult)
{
    // FP8_MAX = 1.75 * 2^kMaxExp for both formats (448 and 57344).
    constexpr int kMaxExp = kFmt == FMT_E4M3 ? 8 : 15;
    const float fmax = kFmt == FMT_E4M3 ? 448.0f : 57344.0f;
    const float amax_c = fmaxf(amax, 0x1p-100f);
    if (kPow2) {
        // smallest j with 1.75 * 2^(kMaxExp + j) >= amax_c, from amax_c's bits
        const uint32_t bits = __builtin_bit_cast(uint32_t, amax_c);
        const int e = (int)(bits >> 23) - 127;
        const int j = e - kMaxExp + ((bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
        scale = __builtin_bit_cast(float, (uint32_t)(j + 127) << 23);
        mult = __builtin_bit_cast(float, (uint32_t)(127 - j) << 23);
    } else {
        scale = amax_c / fmax;  // IEEE-rounded divisions (no fast-math)
        mult = fmax / amax_c;
    }
}

template <int kFmt, bool kPow2>
__global__ __launch_bounds__(kThreads) void cast_per_token_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t groups_per_row, int64_t tiles_c, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scales, int64_t ld_s)
{
    const float fmax = kFmt == FMT_E4M3 ? 448.0f : 57344.0f;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int part = lane & (kLanesPerGroup - 1);
    const int64_t tile_r = blockIdx.x / tiles_c;
    const int64_t tile_c = blockIdx.x - tile_r * tiles_c;
    const int64_t row_raw = tile_r * kTileRows + wave * 8 + (lane >> 3);
    // Rows and groups past the end repeat the last valid one (the 8 lanes of
    // a group stay together, so the DPP exchange is unaffected) and store
    // nothing.
    const bool row_ok = row_raw < rows;
    const int64_t row = row_ok ? row_raw : rows - 1;
    const int64_t g0 = tile_c * kTileGroups;

    u32x4 u[kTileGroups][2];
#pragma unroll
    for (int t = 0; t < kTileGroups; ++t) {
        const int64_t gc = min(g0 + t, groups_per_row - 1);
        const u32x4* src = reinterpret_cast<const u32x4*>(x + row * ld_x + gc * 128 + part * 16);
        u[t][0] = __builtin_nontemporal_load(src);
        u[t][1] = __builtin_nontemporal_load(src + 1);
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
        const uint2 c0 = encode8<kFmt>(s0, fmax);
        const uint2 c1 = encode8<kFmt>(s1, fmax);
        const int64_t gc = g0 + t;
        if (row_ok && gc < groups_per_row) {
            *reinterpret_cast<uint4*>(q + row * ld_q + gc * 128 + part * 16) = make_uint4(c0.x, c0.y, c1.x, c1.y);
            if (part == 0) scales[gc * ld_s + row] = scale;  // block-major: [cols/128][ld_s]
        }
    }
}

}  // namespace

hipError_t launch_cast(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int fmt,
                       bool pow2, uint8_t* q, int64_t ld_q, float* scales, int64_t ld_s, hipStream_t stream,
                       LaunchInfo* info)
{
    const int64_t gpr = cols / 128;
    const int64_t tiles_c = (gpr + kTileGroups - 1) / kTileGroups;
    const int64_t blocks = ((rows + kTileRows - 1) / kTileRows) * tiles_c;
    if (info) { info->tile_m = kTileRows; info->tile_n = 128 * kTileGroups; info->threads = kThreads; info->grid = blocks; }
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (blocks <= 0) return hipSuccess;
    dim3 grid((unsigned)blocks), block(kThreads);
    if (fmt == FMT_E4M3) {
        if (pow2) cast_per_token_kernel<FMT_E4M3, true><<<grid, block, 0, stream>>>(x, rows, gpr, tiles_c, ld_x, q, ld_q, scales, ld_s);
        else cast_per_token_kernel<FMT_E4M3, false><<<grid, block, 0, stream>>>(x, rows, gpr, tiles_c, ld_x, q, ld_q, scales, ld_s);
    } else {
        if (pow2) cast_per_token_kernel<FMT_E5M2, true><<<grid, block, 0, stream>>>(x, rows, gpr, tiles_c, ld_x, q, ld_q, scales, ld_s);
        else cast_per_token_kernel<FMT_E5M2, false><<<grid, block, 0, stream>>>(x, rows, gpr, tiles_c, ld_x, q, ld_q, scales, ld_s);
    }
    return hipGetLastError();
}

}  // namespace tefp8
