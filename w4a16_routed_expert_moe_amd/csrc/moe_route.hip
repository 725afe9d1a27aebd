// moe_route.hip -- router of the MoE layer on gfx950.
//
// The pages fix only that the router has an FP32 gate bias (model card
// "canada-quant/DeepSeek-V4-Flash-W4A16-FP8-MTP", "Component precisions", and
// "Upstream contributions" where its silent downcast to BF16 is a bug) and
// that six of 256 routed experts are active per token ("DeepSeek V4 Flash
// serving hardware", 01, "Sparse architecture").  The expert choice is an
// integer decided by floating point, so the arithmetic here is fixed to the
// last bit and reproducible on any IEEE machine:
//   * logits: 64 lane partials, lane l accumulates elements 512j + 8l + u with
//     fused multiply-add, then a butterfly over lane distance 32..1;
//   * sigmoid through this file's own fp32 exp (Cody-Waite reduction,
//     degree-7 Taylor polynomial), IEEE division;
//   * key = score + bias, top-k by a wavefront bitonic selection over
//     (key, expert) packed into 64-bit words, ties to the lower index;
//   * weights renormalised over the chosen unbiased scores, summed in slot
//     order.
#include "moe_common.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

// ------------------------------------------------------------------ exp
constexpr double kLn2 = 0.693147180559945309417232121458;
constexpr float kLog2e = (float)(1.0 / kLn2);
constexpr float kLn2Hi = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, (float)kLn2) & 0xFFFFF000u);
constexpr float kLn2Lo = (float)(kLn2 - (double)kLn2Hi);
constexpr float kC2 = (float)(1.0 / 2.0), kC3 = (float)(1.0 / 6.0), kC4 = (float)(1.0 / 24.0);
constexpr float kC5 = (float)(1.0 / 120.0), kC6 = (float)(1.0 / 720.0), kC7 = (float)(1.0 / 5040.0);

// e^y: y = n ln2 + r (ln2 split into a 12-bit head and a tail so n*head is
// exact), e^r by its Taylor polynomial to degree 7 (error r^8/8! < 5.2e-9),
// then scaled by 2^n.  Saturates to +inf at y >= 88.5 and to +0 at y <= -86.
__device__ __forceinline__ float exp_f32(float y) {
    if (y >= 88.5f) return __builtin_inff();
    if (y <= -86.0f) return 0.0f;
    const float n = __builtin_rintf(y * kLog2e);
    float r = __builtin_fmaf(-n, kLn2Hi, y);
    r = __builtin_fmaf(-n, kLn2Lo, r);
    float p = kC7;
    p = __builtin_fmaf(p, r, kC6);
    p = __builtin_fmaf(p, r, kC5);
    p = __builtin_fmaf(p, r, kC4);
    p = __builtin_fmaf(p, r, kC3);
    p = __builtin_fmaf(p, r, kC2);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return __builtin_ldexpf(p, (int)n);
}

__device__ __forceinline__ float sigmoid_f32(float l) {
    const float d = 1.0f + exp_f32(-l);
    return __fdiv_rn(1.0f, d);
}

// ------------------------------------------------------------------ logits
// Block = WPB waves; wave w owns tokens t0 + w*TT .. +TT and experts
// [e0, e0+EB).  Each lane keeps its 8*HJ activation elements of each token
// in fp32 registers and streams the router rows.
template <int HJ, int TT>
__global__ __launch_bounds__(256) void k_router_logits(const uint16_t *__restrict__ x,
                                                       const uint16_t *__restrict__ wr,
                                                       float *__restrict__ logits, int T, int E,
                                                       int EB) {
    constexpr int H = HJ * 512;
    const int wave = threadIdx.x >> 6;
    const int l = lane_id();
    const int wpb = blockDim.x >> 6;
    const int t0 = (blockIdx.x * wpb + wave) * TT;
    if (t0 >= T) return;
    const int e0 = blockIdx.y * EB;
    const int e1 = min(E, e0 + EB);

    float xf[TT][HJ][8];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int t = t0 + tt;
#pragma unroll
        for (int j = 0; j < HJ; ++j) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (t < T) v = *(const u32x4 *)(x + (size_t)t * H + 512 * j + 8 * l);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                xf[tt][j][2 * q] = bf16lo_to_f32(v[q]);
                xf[tt][j][2 * q + 1] = bf16hi_to_f32(v[q]);
            }
        }
    }
    for (int e = e0; e < e1; ++e) {
        u32x4 wv[HJ];
#pragma unroll
        for (int j = 0; j < HJ; ++j) wv[j] = *(const u32x4 *)(wr + (size_t)e * H + 512 * j + 8 * l);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            float P = 0.0f;
#pragma unroll
            for (int j = 0; j < HJ; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    P = __builtin_fmaf(xf[tt][j][2 * q], bf16lo_to_f32(wv[j][q]), P);
                    P = __builtin_fmaf(xf[tt][j][2 * q + 1], bf16hi_to_f32(wv[j][q]), P);
                }
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) P = P + __shfl_xor(P, d, kWave);
            const int t = t0 + tt;
            if (l == 0 && t < T) logits[(size_t)t * E + e] = P;
        }
    }
}

// ------------------------------------------------------------------ select
// Orderable 64-bit word: larger key first, then lower expert index.
__device__ __forceinline__ uint64_t pack_key(float key, int e) {
    uint32_t u = __float_as_uint(key);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ void ce_desc(uint64_t &a, uint64_t &b) {  // a >= b afterwards
    const uint64_t hi = a > b ? a : b;
    const uint64_t lo = a > b ? b : a;
    a = hi;
    b = lo;
}

// Sort a bitonic sequence of 8 into descending order.
__device__ __forceinline__ void bitonic_merge8(uint64_t c[8]) {
#pragma unroll
    for (int d = 4; d >= 1; d >>= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if ((i & d) == 0) ce_desc(c[i], c[i + d]);
}

// One wave per token.  Lane l holds experts 4l..4l+3.  Steps: sort the four
// in-lane, merge with lane l^1 into a sorted 8, then five butterfly rounds
// (lane distance 2..32) each keeping the top 8 of two sorted 8-lists (the
// element-wise max of one list and the other reversed is bitonic and holds
// the top 8), so every lane ends with the global top 8 in order.
__global__ __launch_bounds__(256) void k_route_select(const float *__restrict__ logits,
                                                      const float *__restrict__ bias, int T, int E,
                                                      int k, float routed_scale,
                                                      int32_t *__restrict__ topk_idx,
                                                      float *__restrict__ topk_w) {
    const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (t >= T) return;
    const int l = lane_id();
    const float *lg = logits + (size_t)t * E;

    uint64_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = 4 * l + i;
        v[i] = 0;  // below every real key
        if (e < E) v[i] = pack_key(sigmoid_f32(lg[e]) + bias[e], e);
    }
    ce_desc(v[0], v[1]);
    ce_desc(v[2], v[3]);
    ce_desc(v[0], v[2]);
    ce_desc(v[1], v[3]);
    ce_desc(v[1], v[2]);

    uint64_t c[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        c[i] = v[i];
        c[7 - i] = shfl_xor_u64(v[i], 1);
    }
    bitonic_merge8(c);
#pragma unroll
    for (int d = 2; d < kWave; d <<= 1) {
        uint64_t p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = shfl_xor_u64(c[i], d);
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = c[i] > p[7 - i] ? c[i] : p[7 - i];
        bitonic_merge8(c);
    }

    uint64_t mine = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (l == j) mine = c[j];
    int e_sel = 0;
    float s_sel = 0.0f;
    if (l < k) {
        e_sel = (int)(0xFFFFFFFFu - (uint32_t)mine);
        s_sel = sigmoid_f32(lg[e_sel]);
    }
    float S = __shfl(s_sel, 0, kWave);
    for (int j = 1; j < k; ++j) S = S + __shfl(s_sel, j, kWave);
    if (l < k) {
        topk_idx[(size_t)t * k + l] = e_sel;
        topk_w[(size_t)t * k + l] = __fdiv_rn(s_sel, S) * routed_scale;
    }
}

template <int HJ>
void launch_logits(const uint16_t *x, const uint16_t *wr, float *logits, int T, int E,
                   hipStream_t st) {
    constexpr int TT = 2;
    const int wpb = T <= TT ? 1 : 4;
    const int EB = T <= 64 ? 1 : 16;
    dim3 grid((T + wpb * TT - 1) / (wpb * TT), (E + EB - 1) / EB);
    hipLaunchKernelGGL((k_router_logits<HJ, TT>), grid, dim3(64 * wpb), 0, st, x, wr, logits, T, E,
                       EB);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_route(const moe_layer_desc *desc, int32_t T, const uint16_t *x,
                                const uint16_t *w_router, const float *gate_bias, float *logits,
                                int32_t *topk_idx, float *topk_w, void *stream) {
    MOE_TRY(check_desc(desc));
    MOE_TRY(check_tokens(T));
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !gate_bias || !logits || !topk_idx || !topk_w) return MOE_ERR_NULL;
    if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(gate_bias, 4) || !aligned(logits, 4) ||
        !aligned(topk_idx, 4) || !aligned(topk_w, 4))
        return MOE_ERR_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    const int H = desc->hidden, E = desc->n_routed;
    switch (H / 512) {
        case 1: launch_logits<1>(x, w_router, logits, T, E, st); break;
        case 2: launch_logits<2>(x, w_router, logits, T, E, st); break;
        case 4: launch_logits<4>(x, w_router, logits, T, E, st); break;
        case 8: launch_logits<8>(x, w_router, logits, T, E, st); break;
        default: return MOE_ERR_UNSUPPORTED;
    }
    MOE_TRY(launch_status());
    hipLaunchKernelGGL(k_route_select, dim3((T + 3) / 4), dim3(256), 0, st, logits, gate_bias, T, E,
                       desc->top_k, desc->routed_scale, topk_idx, topk_w);
    return launch_status();
}
