// moe_gemm_common.h -- what the two grouped W4A16 GEMM kernels share: the
// INT4 unpack, the MFMA wrapper, the launch arguments, and the entry to the
// tiled kernel (moe_gemm_tiled.hip, compiled with its own scheduling flags).
#pragma once

#include "moe_common.h"

namespace moe {

constexpr uint32_t kMagic = 0x43004300u;  // bf16 128.0 in both halves
constexpr uint16_t kNeg136 = 0xC308;      // bf16 -136.0

// (x & 0x000F000F) | kMagic as one v_bitop3 (truth table 0xEA = (a & b) | c);
// written as two operations the compiler emits an AND and an OR with literals
__device__ __forceinline__ uint32_t nib_to_bf16x2(uint32_t x) {
    return __builtin_amdgcn_bitop3_b32(x, 0x000F000Fu, kMagic, 0xEA);
}

__device__ __forceinline__ bf16x8 unpack_codes(uint32_t w) {
    u32x4 r;
    r[0] = nib_to_bf16x2(w);
    r[1] = nib_to_bf16x2(w >> 4);
    r[2] = nib_to_bf16x2(w >> 8);
    r[3] = nib_to_bf16x2(w >> 12);
    return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

struct GemmArgs {
    const uint16_t *a;
    const int32_t *gather;
    int n_src;
    const u32x4 *wq;
    const void *scales;  // fp16 [G][N][K/128] (INT4) or UE8M0 bytes [G][N][K/32] (FP4)
    const int32_t *offsets;
    int G, R, N, K;
    uint16_t *out;
    bool single;        // every group fits one work item
    const float *sums;  // row sums of a over 128-wide k groups, or null
};

// The tiled kernel takes groups with many rows: T >= 256 tokens, N a
// multiple of its 128-row n-block, K at most 4096 (its scale table in LDS).
bool use_tiled(int T, int N, int K, int act);  // from MOE_TILED_MIN_TOKENS(_NOACT), ...
void launch_tiled(int act, const GemmArgs &p, hipStream_t st, bool fp4 = false);

}  // namespace moe
