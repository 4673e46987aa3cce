// Internal interface between the C-ABI front end (api.cpp) and the gfx950
// kernels (cast.hip, gemm.hip).  Not installed; not part of the ABI.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace tefp8 {

// fp8 operand format as the matrix-core instruction encodes it (cbsz/blgp).
enum Fmt : int { FMT_E4M3 = 0, FMT_E5M2 = 1 };

enum class Epi : int {
    Wgrad = 0,  // out[m][n] += acc (fp32 read-modify-write)
    Fwd = 1,    // bias / GELU / aux pre-activation, bf16 or fp32 store
    Dgrad = 2   // dGELU / bias-gradient, bf16 or fp32 store
};

// One contraction group (dense GEMMs have exactly one).
struct Group {
    int32_t kb_off;   // first 128-column block of the group
    int32_t kb_len;   // number of 128-column blocks (>= 1)
    int32_t out_idx;  // which output matrix (out + out_idx * out_group_stride)
    int32_t pad;
};

constexpr int kMaxGroupsPerLaunch = 128;
constexpr int kMaxDeviceGroups = 256;  // groups of the device-sized K-grouped call
constexpr int kMGroupRows = 256;       // rows per block of the M-grouped layout (the GEMM's tile height)

struct GemmArgs {
    const uint8_t* a;      // [M][lda] fp8
    const float* sa;       // [K/128][lsa]
    const uint8_t* b;      // [N][ldb] fp8
    const float* sb;       // [K/128][lsb]
    int64_t M, N;
    int64_t lda, ldb;      // bytes
    int64_t lsa, lsb;      // floats between consecutive 128-deep blocks of sa / sb (block-major scales)
    int fmt_a, fmt_b;      // Fmt
    bool fast;             // accumulation policy
    Epi epi;
    uint32_t flags;        // TE_EPI_* bits
    // outputs
    void* out;             // fp32 (wgrad / f32 store) or bf16
    bool out_bf16;
    int64_t ld_out;        // elements
    int64_t out_group_stride;  // elements between consecutive out matrices (grouped)
    const uint16_t* bias;  // [N] bf16 (Fwd)
    uint16_t* aux;         // [M][ld_aux] bf16 pre-activation store (Fwd)
    const uint16_t* preact;  // [M][ld_aux] bf16 (Dgrad)
    int64_t ld_aux;
    float* bias_grad;      // [N] (Dgrad)
    // groups
    int num_groups;
    Group groups[kMaxGroupsPerLaunch];
    // K-grouped with group sizes in device memory: when set, groups[] is
    // unused, group g's contraction range is read from group_k_dev (K per
    // group, in elements) and clamped to the sum_kb blocks of the operands.
    const int64_t* group_k_dev;
    int64_t sum_kb;
    // M-grouped (mixture-of-experts forward/data gradient): when set, the
    // 256-row block i of A belongs to expert m_block_group[i] (device memory;
    // a value outside [0, num_b_groups) skips the block, its output rows are
    // not written), whose B operand, B scales and bias sit at these strides.
    const int32_t* m_block_group;
    int32_t num_b_groups;
    int64_t b_group_stride;     // bytes
    int64_t sb_group_stride;    // floats
    int64_t bias_group_stride;  // elements
    // Quantising forward store: when q_out is set the forward epilogue writes
    // the per-token cast of its fp32 result (groups of 128 columns) instead
    // of y: codes [M][ld_q], scales block-major [N/128][ld_qs].
    uint8_t* q_out;
    float* q_scales;
    int64_t ld_q, ld_qs;
    int q_fmt;
    int q_pow2;
    // ... and/or the cast of its transpose (groups of 128 rows, the weight
    // gradient's along-tokens operand): codes [N][ld_qt], scales block-major
    // [M/128][ld_qts].  Either q_out or qt_out (or both) is set.
    uint8_t* qt_out;
    float* qt_scales;
    int64_t ld_qt, ld_qts;
    // Deterministic bias gradient: when set, each wave stores its column sums
    // to row (tile_m * 4 + wave_m) of this [P][bgrad_ws_ld] workspace instead
    // of adding them atomically; a second kernel sums the rows in order.
    float* bgrad_ws;
    int64_t bgrad_ws_ld;
};

struct LaunchInfo {
    int tile_m, tile_n, threads;
    int64_t grid;
};

int device_cus();  // compute units of the current device
hipError_t launch_gemm(const GemmArgs& args, hipStream_t stream, LaunchInfo* info);
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t stream);
// bias_grad[n] = sum over p = 0 .. rows-1, in order, of ws[p * ld + n]
hipError_t launch_bgrad_reduce(const float* ws, int64_t rows, int64_t ld, int64_t N, float* bias_grad,
                               hipStream_t stream);
constexpr int kBgradRowsPerTile = 4;  // waves along M per 256-row tile
// bias_grad[e][n] = sum over the 256-row blocks b with m_block_group[b] == e,
// in order, of their kBgradRowsPerTile workspace rows (G experts, [G][N] out)
hipError_t launch_mgrouped_bgrad_reduce(const float* ws, int64_t blocks, int64_t ld, int64_t N, int32_t G,
                                        const int32_t* m_block_group, float* bias_grad, hipStream_t stream);
// Device address of the library's static scratch array on the current device
// (looked up once per device, then cached); its size is TE_NOALLOC_SCRATCH_BYTES.
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_cast(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int fmt,
                       bool pow2, uint8_t* q, int64_t ld_q, float* scales, int64_t ld_s, hipStream_t stream,
                       LaunchInfo* info);
// One operand of a batched per-token cast (gpr, tiles_c and tile_begin are
// filled in by launch_cast_batch).
struct CastOperand {
    const uint16_t* x;
    int64_t rows, cols, ld_x;
    uint8_t* q;
    int64_t ld_q;
    float* scales;
    int64_t ld_s;
    int64_t gpr, tiles_c, tile_begin;
};
constexpr int kMaxCastBatch = 8;
struct CastBatch {
    int n;
    CastOperand op[kMaxCastBatch];
};
// out[r] = sum over k of the dequantised fp8 operand row r (block-major scales)
hipError_t launch_row_sum(const uint8_t* q, int64_t rows, int64_t cols, int64_t ld_q, int fmt, const float* scales,
                          int64_t ld_s, float* out, hipStream_t stream);
hipError_t launch_cast_batch(const CastOperand* ops, int n, int fmt, bool pow2, hipStream_t stream, LaunchInfo* info);
// Row-wise cast (q may be null) and cast of the transpose in one pass; rows a
// multiple of 128, cols a multiple of 128 with the row-wise cast, else of 8.
hipError_t launch_cast_transpose(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int fmt, bool pow2,
                                 uint8_t* q, int64_t ld_q, float* scales, int64_t ld_s, uint8_t* qt, int64_t ld_qt,
                                 float* scales_t, int64_t ld_st, hipStream_t stream, LaunchInfo* info);

}  // namespace tefp8
