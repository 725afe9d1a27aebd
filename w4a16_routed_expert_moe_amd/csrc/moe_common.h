// moe_common.h -- shared device/host helpers of the gfx950 MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_w4a16.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf16lo_to_f32(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (the conversion of the __bf16 type).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int d) {
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    lo = __shfl_xor(lo, d, kWave);
    hi = __shfl_xor(hi, d, kWave);
    return ((uint64_t)hi << 32) | lo;
}

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ int wave_incl_scan(int v) {
    const int l = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int o = __shfl_up(v, d, kWave);
        if (l >= d) v += o;
    }
    return v;
}

// ---------------------------------------------------------------- host side
inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline moe_status check_desc(const moe_layer_desc *d) {
    if (!d) return MOE_ERR_NULL;
    if (d->hidden != 512 && d->hidden != 1024 && d->hidden != 2048 && d->hidden != 4096)
        return MOE_ERR_SHAPE;
    if (d->inter < 128 || d->inter > 4096 || d->inter % 128) return MOE_ERR_SHAPE;
    {   // inter/128 must split evenly into <= 4 slices of 1, 2, 4 or 8 k groups
        const int kg = d->inter / 128;
        bool ok = false;
        for (int kgw = 1; kgw <= 8; kgw *= 2) ok = ok || (kg % kgw == 0 && kg / kgw <= 4);
        if (!ok) return MOE_ERR_SHAPE;
    }
    if (d->n_routed < 1 || d->n_routed > 256) return MOE_ERR_SHAPE;
    if (d->top_k < 1 || d->top_k > 8 || d->top_k > d->n_routed) return MOE_ERR_SHAPE;
    if (d->n_shared != 0 && d->n_shared != 1) return MOE_ERR_SHAPE;
    if (d->group_size != 128) return MOE_ERR_UNSUPPORTED;
    if (!(d->routed_scale == d->routed_scale) || d->routed_scale > 3.0e38f || d->routed_scale < -3.0e38f)
        return MOE_ERR_SHAPE;
    return MOE_OK;
}

inline moe_status check_tokens(int32_t T) {
    if (T < 0 || T > MOE_MAX_TOKENS) return MOE_ERR_SHAPE;
    return MOE_OK;
}

inline moe_status launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

// Caller workspace of moe_permute / moe_route_permute (moe_workspace_bytes):
// a 256-byte header (int32 word 0: moe_route_permute's counter for T <= 4,
// zero between calls), then, past one chunk of 1024 tokens, the permutation's
// per-chunk table int32 [chunks][320].
constexpr size_t kWsHeaderBytes = 256;
size_t workspace_bytes(const moe_layer_desc *desc, int32_t T);
moe_status check_workspace(const moe_layer_desc *desc, int32_t T, const void *ws, size_t ws_bytes);
moe_status launch_permute(const moe_layer_desc *desc, int32_t T, const int32_t *topk_idx,
                          int32_t *group_offsets, int32_t *sorted_token, int32_t *row_of_slot,
                          void *ws, hipStream_t st);

#define MOE_TRY(expr)                      \
    do {                                   \
        moe_status _s = (expr);            \
        if (_s != MOE_OK) return _s;       \
    } while (0)

}  // namespace moe
