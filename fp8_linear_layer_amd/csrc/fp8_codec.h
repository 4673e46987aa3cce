// fp8 codec pieces shared by the per-token cast kernels and the quantising
// GEMM epilogue (device code only): the group scale and the RNE encoding of
// eight fp32 values.  The reading of the per-token cast is the one in
// te_fp8.h: s = fl32(amax_c / FP8_MAX), codes enc(fl32(x * fl32(FP8_MAX /
// amax_c))), amax_c = max(amax, 2^-100); or the power of two just above.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace tefp8 {

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

// Eight fp32 values (already scaled) -> eight fp8 codes in two dwords: the
// hardware v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 (round to nearest even) on
// inputs clamped to +-FP8_MAX (the clamp gives saturation).
template <int kFmt>
__device__ __forceinline__ uint2 encode8(const float (&v)[8])
{
    const float fmax = kFmt == FMT_E4M3 ? 448.0f : 57344.0f;
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

}  // namespace tefp8
