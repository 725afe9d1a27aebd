// moe_combine.hip -- weighted combine of the expert outputs on gfx950.
//
// out[t] = bf16( y[shared row of t] + sum_j w[t][j] * y[row of slot (t, j)] ):
// the shared expert is always on with weight 1 and the k routed outputs are
// weighted by the renormalised router weights ("DeepSeek V4 Flash serving
// hardware", 01, "Sparse architecture": one shared plus six routed experts
// per token).  Each thread owns 8 consecutive hidden elements (16-byte loads
// and stores), sums in fp32 in slot order, and writes each output once, so
// the result is deterministic (no atomics).
#include "moe_common.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void k_combine(const uint16_t *__restrict__ y,
                                                 const int32_t *__restrict__ row_of_slot,
                                                 const float *__restrict__ topk_w, int T, int H,
                                                 int k, int ns, int R, uint16_t *__restrict__ out) {
    const int t = blockIdx.x;
    const int h0 = (blockIdx.y * blockDim.x + threadIdx.x) * 8;
    if (t >= T || h0 >= H) return;
    const int S = k + ns;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    if (ns) {
        const int r = row_of_slot[(size_t)t * S + k];
        if ((unsigned)r < (unsigned)R) {
            const u32x4 v = *(const u32x4 *)(y + (size_t)r * H + h0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = bf16lo_to_f32(v[q]);
                acc[2 * q + 1] = bf16hi_to_f32(v[q]);
            }
        }
    }
    for (int j = 0; j < k; ++j) {
        const int r = row_of_slot[(size_t)t * S + j];
        const float w = topk_w[(size_t)t * k + j];
        if ((unsigned)r >= (unsigned)R) continue;
        const u32x4 v = *(const u32x4 *)(y + (size_t)r * H + h0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[2 * q] = __builtin_fmaf(w, bf16lo_to_f32(v[q]), acc[2 * q]);
            acc[2 * q + 1] = __builtin_fmaf(w, bf16hi_to_f32(v[q]), acc[2 * q + 1]);
        }
    }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    *(u32x4 *)(out + (size_t)t * H + h0) = o;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_combine(const moe_layer_desc *desc, int32_t T, const uint16_t *y,
                                  const int32_t *row_of_slot, const float *topk_w, uint16_t *out,
                                  void *stream) {
    MOE_TRY(check_desc(desc));
    MOE_TRY(check_tokens(T));
    if (T == 0) return MOE_OK;
    if (!y || !row_of_slot || !topk_w || !out) return MOE_ERR_NULL;
    if (!aligned(y, 16) || !aligned(row_of_slot, 4) || !aligned(topk_w, 4) || !aligned(out, 16))
        return MOE_ERR_ALIGN;
    const int H = desc->hidden;
    const int R = T * (desc->top_k + desc->n_shared);
    dim3 grid(T, (H / 8 + 255) / 256);
    hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, (hipStream_t)stream, y, row_of_slot, topk_w, T,
                       H, desc->top_k, desc->n_shared, R, out);
    return launch_status();
}
