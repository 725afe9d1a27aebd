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

// The router's lane reduction: partial l becomes P_l + P_{l^d} for
// d = 32, 16, 8, 4, 2, 1, every lane ending with the same sum.  Levels 32 and
// 16 swap half-waves or row pairs between two copies and add (fp32 addition
// commutes, so both lanes of a pair get the same value); levels 8..1 add the
// value rotated by d within each 16-lane row, which equals the value at l^d
// because after the level above the row is periodic in 2d.  No LDS traffic.
__device__ __forceinline__ float wave_tree_sum(float P) {
    {
        const uint32_t a = __float_as_uint(P);
        const auto r = __builtin_amdgcn_permlane32_swap(a, a, false, false);
        P = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    {
        const uint32_t a = __float_as_uint(P);
        const auto r = __builtin_amdgcn_permlane16_swap(a, a, false, false);
        P = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
#define MOE_ROR_ADD(CTRL) \
    P = P + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, P), CTRL, 0xF, 0xF, false))
    MOE_ROR_ADD(0x128);  // row_ror:8
    MOE_ROR_ADD(0x124);  // row_ror:4
    MOE_ROR_ADD(0x122);  // row_ror:2
    MOE_ROR_ADD(0x121);  // row_ror:1
#undef MOE_ROR_ADD
    return P;
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
    // the next expert's router row is loaded while this one is used
    u32x4 wn[HJ];
#pragma unroll
    for (int j = 0; j < HJ; ++j) wn[j] = *(const u32x4 *)(wr + (size_t)e0 * H + 512 * j + 8 * l);
    for (int e = e0; e < e1; ++e) {
        u32x4 wv[HJ];
#pragma unroll
        for (int j = 0; j < HJ; ++j) wv[j] = wn[j];
        const int en = min(e + 1, e1 - 1);
#pragma unroll
        for (int j = 0; j < HJ; ++j) wn[j] = *(const u32x4 *)(wr + (size_t)en * H + 512 * j + 8 * l);
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
            P = wave_tree_sum(P);
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

// Exchange with the partner lane of a merge level.  The partner only has to
// sit in the other half of the group being merged, so the within-row levels
// use DPP lane permutes (VALU latency): quad permutes for distance 1 and 2,
// row_half_mirror (l <-> 7-l) and row_mirror (l <-> 15-l) for the 8- and
// 16-lane groups; the 32- and 64-lane levels go through the LDS crossbar.
template <int D>
__device__ __forceinline__ uint32_t xchg32(uint32_t v) {
    if constexpr (D == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
    if constexpr (D == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
    if constexpr (D == 4) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);
    if constexpr (D == 8) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false);
    return __shfl_xor(v, D, kWave);
}

template <int D>
__device__ __forceinline__ uint64_t xchg64(uint64_t v) {
    const uint32_t lo = xchg32<D>((uint32_t)v), hi = xchg32<D>((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Sort a bitonic sequence of 8 into descending order.
__device__ __forceinline__ void bitonic_merge8(uint64_t c[8]) {
#pragma unroll
    for (int d = 4; d >= 1; d >>= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if ((i & d) == 0) ce_desc(c[i], c[i + d]);
}

// Keep the top 8 of this lane's sorted list and its partner's (level D).
template <int D>
__device__ __forceinline__ void merge_top8(uint64_t c[8]) {
    uint64_t p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = xchg64<D>(c[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = c[i] > p[7 - i] ? c[i] : p[7 - i];
    bitonic_merge8(c);
}

// One wave selects for one token (logits lg[0..E)).  Lane l holds experts
// 4l..4l+3.  Steps: sort the four in-lane, merge with lane l^1 into a sorted
// 8, then five rounds (groups of 4, 8, 16, 32, 64 lanes) each keeping the top 8
// of two sorted 8-lists (the element-wise max of one list and the other
// reversed is bitonic and holds the top 8), so every lane ends with the
// global top 8 in order.  Lanes j < k write slot j; lane j returns its expert.
__device__ __forceinline__ int select_token(const float *__restrict__ lg,
                                            const float *__restrict__ bias, int E, int k,
                                            float routed_scale, int32_t *__restrict__ idx_out,
                                            float *__restrict__ w_out) {
    const int l = lane_id();
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
        c[7 - i] = xchg64<1>(v[i]);
    }
    bitonic_merge8(c);
    merge_top8<2>(c);
    merge_top8<4>(c);
    merge_top8<8>(c);
    merge_top8<16>(c);
    merge_top8<32>(c);

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
        idx_out[l] = e_sel;
        w_out[l] = __fdiv_rn(s_sel, S) * routed_scale;
    }
    return e_sel;
}

__global__ __launch_bounds__(256) void k_route_select(const float *__restrict__ logits,
                                                      const float *__restrict__ bias, int T, int E,
                                                      int k, float routed_scale,
                                                      int32_t *__restrict__ topk_idx,
                                                      float *__restrict__ topk_w) {
    const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (t >= T) return;
    select_token(logits + (size_t)t * E, bias, E, k, routed_scale, topk_idx + (size_t)t * k,
                 topk_w + (size_t)t * k);
}

// ------------------------------------------------------------------ fused
// Stable counting sort of the T*(k+ns) <= 64 slots of a small batch by one
// wave, with no cross-lane traffic: lane f owns slot f = t*(k+ns) + j, its row
// is (slots in lower groups) + (earlier slots of its group), and
// group_offsets[g] is the number of slots in groups below g.
__device__ __forceinline__ void permute_small(const int *__restrict__ idx_lds, int T, int E, int k,
                                              int ns, int *g_lds, int32_t *__restrict__ offsets,
                                              int32_t *__restrict__ sorted_token,
                                              int32_t *__restrict__ row_of_slot) {
    const int l = lane_id();
    const int S = k + ns, nslot = T * S, G = E + ns;
    int g = -1, t = 0, j = 0;
    if (l < nslot) {
        t = l / S;
        j = l - t * S;
        g = j < k ? min(max(idx_lds[t * k + j], 0), E - 1) : E;
    }
    g_lds[l] = g;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int below[5] = {0, 0, 0, 0, 0};  // groups 5l..5l+4 (G <= 257 < 320)
    int pos = 0;
    for (int f = 0; f < nslot; ++f) {
        const int gf = g_lds[f];
#pragma unroll
        for (int i = 0; i < 5; ++i) below[i] += gf < 5 * l + i;
        pos += gf < g || (gf == g && f < l);
    }
#pragma unroll
    for (int i = 0; i < 5; ++i)
        if (5 * l + i <= G) offsets[5 * l + i] = below[i];
    if (l < nslot) {
        sorted_token[pos] = t;
        row_of_slot[t * S + j] = pos;
    }
}

// Route and permute a batch of T <= 4 tokens in one launch.  Each wave
// computes one expert's logits for every token and publishes them with
// device-coherent stores; the workgroup whose increment of `sync` comes last
// reads them back with device-coherent loads, selects the top k of each token
// (one wave per token) and sorts the slots, then returns the counter to zero
// for the next call.
template <int HJ, int TT>
__global__ __launch_bounds__(256) void k_route_permute_small(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr, const float *__restrict__ bias,
    int T, int E, int k, int ns, float routed_scale, float *__restrict__ logits,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, int32_t *__restrict__ offsets,
    int32_t *__restrict__ sorted_token, int32_t *__restrict__ row_of_slot, int32_t *sync) {
    constexpr int H = HJ * 512;
    __shared__ int s_last;
    __shared__ int idx_lds[4 * 8];
    __shared__ int g_lds[kWave];
    __shared__ float lg_lds[4][256];
    const int wave = threadIdx.x >> 6;
    const int l = lane_id();
    const int e = blockIdx.x * 4 + wave;
    if (e < E) {
        u32x4 xv[TT][HJ];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int j = 0; j < HJ; ++j) {
                xv[tt][j] = u32x4{0u, 0u, 0u, 0u};
                if (tt < T) xv[tt][j] = *(const u32x4 *)(x + (size_t)tt * H + 512 * j + 8 * l);
            }
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
                    P = __builtin_fmaf(bf16lo_to_f32(xv[tt][j][q]), bf16lo_to_f32(wv[j][q]), P);
                    P = __builtin_fmaf(bf16hi_to_f32(xv[tt][j][q]), bf16hi_to_f32(wv[j][q]), P);
                }
            P = wave_tree_sum(P);
            // device-coherent (write-through) store: visible to every XCD once
            // the store has completed, without writing back the whole L2
            if (l == 0 && tt < T)
                __hip_atomic_store(logits + (size_t)tt * E + e, P, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's logit stores have completed
    __syncthreads();
    if (threadIdx.x == 0)
        s_last = __hip_atomic_fetch_add(sync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 (int)gridDim.x - 1;
    __syncthreads();
    if (!s_last) return;
    // every other workgroup's stores completed before its increment; read the
    // logits with device-coherent loads (no stale L2 line can answer)
    for (int i = threadIdx.x; i < T * E; i += blockDim.x)
        lg_lds[i / E][i % E] =
            __hip_atomic_load(logits + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (wave < T) {
        const int es = select_token(lg_lds[wave], bias, E, k, routed_scale,
                                    topk_idx + (size_t)wave * k, topk_w + (size_t)wave * k);
        if (l < k) idx_lds[wave * k + l] = es;
    }
    __syncthreads();
    if (wave == 0) permute_small(idx_lds, T, E, k, ns, g_lds, offsets, sorted_token, row_of_slot);
    if (threadIdx.x == 0) __hip_atomic_exchange(sync, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

template <int HJ>
static void launch_small(const moe_layer_desc *d, int T, const uint16_t *x, const uint16_t *wr,
                         const float *bias, float *logits, int32_t *topk_idx, float *topk_w,
                         int32_t *offsets, int32_t *sorted_token, int32_t *row_of_slot,
                         int32_t *sync, hipStream_t st) {
    const dim3 grid((d->n_routed + 3) / 4);
#define MOE_SMALL(TT)                                                                              \
    hipLaunchKernelGGL((k_route_permute_small<HJ, TT>), grid, dim3(256), 0, st, x, wr, bias, T,      \
                       d->n_routed, d->top_k, d->n_shared, d->routed_scale, logits, topk_idx,    \
                       topk_w, offsets, sorted_token, row_of_slot, sync)
    if (T == 1)
        MOE_SMALL(1);
    else if (T == 2)
        MOE_SMALL(2);
    else
        MOE_SMALL(4);
#undef MOE_SMALL
}

extern "C" moe_status moe_route_permute(const moe_layer_desc *desc, int32_t T, const uint16_t *x,
                                        const uint16_t *w_router, const float *gate_bias,
                                        float *logits, int32_t *topk_idx, float *topk_w,
                                        int32_t *group_offsets, int32_t *sorted_token,
                                        int32_t *row_of_slot, int32_t *sync, void *stream) {
    MOE_TRY(check_desc(desc));
    MOE_TRY(check_tokens(T));
    if (T == 0) return MOE_OK;
    if (T > 4) {
        MOE_TRY(moe_route(desc, T, x, w_router, gate_bias, logits, topk_idx, topk_w, stream));
        return moe_permute(desc, T, topk_idx, group_offsets, sorted_token, row_of_slot, stream);
    }
    if (!x || !w_router || !gate_bias || !logits || !topk_idx || !topk_w || !group_offsets ||
        !sorted_token || !row_of_slot || !sync)
        return MOE_ERR_NULL;
    if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(gate_bias, 4) || !aligned(logits, 4) ||
        !aligned(topk_idx, 4) || !aligned(topk_w, 4) || !aligned(group_offsets, 4) ||
        !aligned(sorted_token, 4) || !aligned(row_of_slot, 4) || !aligned(sync, 4))
        return MOE_ERR_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    switch (desc->hidden / 512) {
        case 1: launch_small<1>(desc, T, x, w_router, gate_bias, logits, topk_idx, topk_w, group_offsets, sorted_token, row_of_slot, sync, st); break;
        case 2: launch_small<2>(desc, T, x, w_router, gate_bias, logits, topk_idx, topk_w, group_offsets, sorted_token, row_of_slot, sync, st); break;
        case 4: launch_small<4>(desc, T, x, w_router, gate_bias, logits, topk_idx, topk_w, group_offsets, sorted_token, row_of_slot, sync, st); break;
        case 8: launch_small<8>(desc, T, x, w_router, gate_bias, logits, topk_idx, topk_w, group_offsets, sorted_token, row_of_slot, sync, st); break;
        default: return MOE_ERR_UNSUPPORTED;
    }
    return launch_status();
}
