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
//   * key = score + bias, top-k by k rounds of a wavefront maximum over
//     (key, expert) packed into 64-bit words, ties to the lower index;
//   * weights renormalised over the chosen unbiased scores, summed in slot
//     order.
#include <mutex>
#include <type_traits>

#include "moe_gemm_common.h"

#include "moe_route_common.h"

namespace moe {
namespace {

using namespace route;

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

// Logits of large batches.  A workgroup of BT/4 waves takes a block of BT
// tokens x 16 experts, wave (wt, we) the 8 x 8 sub-block of tokens
// t0 + 8wt.. and experts e0 + 8we..  Per 512-wide k tile the block's BT
// token rows and 16 router rows (1 KB each) go from global memory straight
// into one of two LDS stages; each lane reads its 16-byte word (elements
// 512j + 8l .. +8) of its 8 token rows and 8 router rows, converts every
// element once and makes 64 fused multiply-adds with it, so a conversion
// serves eight products (two in k_router_logits).  Each (token, expert)
// partial accumulates its lane's elements in the order of router_dot (tile
// j, then element u) and the wave adds the partials by the same tree: the
// logits are k_router_logits' bit for bit.
constexpr int kRbE = 16;  // experts per block
template <int HJ, int BT>
__global__ __launch_bounds__(BT * 16) void k_router_logits_blk(const uint16_t *__restrict__ x,
                                                              const uint16_t *__restrict__ wr,
                                                              float *__restrict__ logits, int T, int E) {
    constexpr int H = HJ * 512;
    constexpr int NW = BT / 4;          // waves: (BT / 8) x 2 sub-blocks of 8 x 8
    constexpr int ROWS = BT + kRbE;     // rows of a tile
    static_assert(ROWS % NW == 0, "rows per wave");
    constexpr int RPW = ROWS / NW;
    __shared__ u32x4 sx[2][BT][kWave], sw[2][kRbE][kWave];  // [stage][row][lane]
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = lane_id();
    const int t0 = blockIdx.x * BT, e0 = blockIdx.y * kRbE;
    const int wt = wave >> 1, we = wave & 1;
    // the block's rows of tile j: wave w moves rows RPW*w .. +RPW (token
    // rows first, then router rows; rows past T or E repeat the last one)
    auto load_tile = [&](int st, int j) {
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int r = RPW * wave + i;
            if (r < BT) {
                const int t = min(t0 + r, T - 1);
                dma16_untracked(x + (size_t)t * H + 512 * j + 8 * l, &sx[st][r][0]);
            } else {
                const int e = min(e0 + r - BT, E - 1);
                dma16_untracked(wr + (size_t)e * H + 512 * j + 8 * l, &sw[st][r - BT][0]);
            }
        }
    };
    float P[8][8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) P[t][e] = 0.0f;
    load_tile(0, 0);
#pragma unroll 1
    for (int j = 0; j < HJ; ++j) {
        const int st = j & 1;
        // this wave's loads of tile j have landed (nothing else is in flight
        // on the vector memory path), and after the barrier every wave's have
        // and every wave is done reading the other stage
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (j + 1 < HJ) load_tile(st ^ 1, j + 1);
        u32x4 xw[8], ww[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) xw[t] = sx[st][8 * wt + t][l];
#pragma unroll
        for (int e = 0; e < 8; ++e) ww[e] = sw[st][8 * we + e][l];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float xf[8], wf[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) xf[t] = h ? bf16hi_to_f32(xw[t][q]) : bf16lo_to_f32(xw[t][q]);
#pragma unroll
                for (int e = 0; e < 8; ++e) wf[e] = h ? bf16hi_to_f32(ww[e][q]) : bf16lo_to_f32(ww[e][q]);
#pragma unroll
                for (int t = 0; t < 8; ++t)
#pragma unroll
                    for (int e = 0; e < 8; ++e) P[t][e] = __builtin_fmaf(xf[t], wf[e], P[t][e]);
            }
    }
    // the 64 sums of the sub-block by wave_tree_sum's tree (lane l added to
    // lane l^32, then l^16, 8, 4, 2, 1), transposed: each level adds every
    // value to its partner lane's copy (addition commutes, so each sum is
    // that tree's bit for bit) and keeps half of them, the half whose index
    // bit matches the lane bit, so that lane l ends with value 8t + e = l
    // (about a third of the instructions of 64 separate trees)
    float v[64];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) v[8 * t + e] = P[t][e];
    // l^32 and l^16: the swap instructions trade the kept half's partner
    // values between the two lanes directly
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 32]), false, false);
        v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 16]), false, false);
        v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    // inside 16-lane rows: the lane with bit d set keeps value i + n/2 and
    // sends value i; the partner's sent value arrives by a lane move
    auto level = [&](int n, int d, auto move) {
        const bool hi = (l & d) != 0;
#pragma unroll
        for (int i = 0; i < n / 2; ++i) {
            const float keep = hi ? v[i + n / 2] : v[i];
            const float send = hi ? v[i] : v[i + n / 2];
            v[i] = keep + move(send, hi);
        }
    };
    auto dpp = [](float x, auto ctrl) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), decltype(ctrl)::value,
                                                                     0xF, 0xF, false));
    };
    using R8 = std::integral_constant<int, 0x128>;   // row_ror:8 (lane l^8)
    using R4 = std::integral_constant<int, 0x124>;   // row_ror:4 (lane l-4 in the row)
    using R12 = std::integral_constant<int, 0x12C>;  // row_ror:12 (lane l+4 in the row)
    using X2 = std::integral_constant<int, 0x4E>;    // quad_perm [2,3,0,1] (lane l^2)
    using X1 = std::integral_constant<int, 0xB1>;    // quad_perm [1,0,3,2] (lane l^1)
    level(16, 8, [&](float x, bool) { return dpp(x, R8()); });
    level(8, 4, [&](float x, bool hi) {
        const float a = dpp(x, R4()), b = dpp(x, R12());
        return hi ? a : b;
    });
    level(4, 2, [&](float x, bool) { return dpp(x, X2()); });
    level(2, 1, [&](float x, bool) { return dpp(x, X1()); });
    const float mine = v[0];
    const int t = t0 + 8 * wt + (l >> 3), e = e0 + 8 * we + (l & 7);
    if (t < T && e < E) logits[(size_t)t * E + e] = mine;
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
            const float P = router_dot<HJ>(xv[tt], wv);
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

// from this many tokens the logits take the block kernel
constexpr int kRouterBlockMinTokens = 512;
// tokens per block: 16 (four waves); 32 on eight waves, which halves the
// re-reads of the router rows, took 359 against 329 us at 8192 tokens

template <int HJ>
void launch_logits(const uint16_t *x, const uint16_t *wr, float *logits, int T, int E,
                   hipStream_t st) {
    if (T >= kRouterBlockMinTokens) {
        constexpr int BT = 16;
        const dim3 grid((T + BT - 1) / BT, (E + kRbE - 1) / kRbE);
        hipLaunchKernelGGL((k_router_logits_blk<HJ, BT>), grid, dim3(BT * 16), 0, st, x, wr, logits, T, E);
        return;
    }
    constexpr int TT = 2;
    const int wpb = T <= TT ? 1 : 4;
    // experts per workgroup: one while the tokens alone give few waves, four
    // at 33..64 tokens (decode64 step 0.275 -> 0.271 ms; 2 or 8: 11.3-11.5
    // against 9.8 us), sixteen above, sixty-four from 4096 tokens, where
    // each wave's activations then serve more rows (8192 tokens: 508 -> 464
    // us; 32 or 128: 475, 468 us; at 2048 tokens 16, 32 and 64 are within 2%)
    const int EB = T <= 32 ? 1 : T <= 64 ? 4 : T < 4096 ? 16 : 64;
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

namespace moe {

// moe_route_permute once the descriptor, T (> 0) and the workspace are
// checked; ws is the caller's workspace or the library's own scratch.
moe_status route_permute(const moe_layer_desc *desc, int32_t T, const uint16_t *x,
                         const uint16_t *w_router, const float *gate_bias, float *logits,
                         int32_t *topk_idx, float *topk_w, int32_t *group_offsets,
                         int32_t *sorted_token, int32_t *row_of_slot, void *ws, hipStream_t st) {
    if (T > 4) {
        MOE_TRY(moe_route(desc, T, x, w_router, gate_bias, logits, topk_idx, topk_w, st));
        if (!group_offsets || !sorted_token || !row_of_slot) return MOE_ERR_NULL;
        if (!aligned(group_offsets, 4) || !aligned(sorted_token, 4) || !aligned(row_of_slot, 4))
            return MOE_ERR_ALIGN;
        return launch_permute(desc, T, topk_idx, group_offsets, sorted_token, row_of_slot, ws, st);
    }
    int32_t *sync = (int32_t *)ws;  // word 0 of the header
    if (!x || !w_router || !gate_bias || !logits || !topk_idx || !topk_w || !group_offsets ||
        !sorted_token || !row_of_slot)
        return MOE_ERR_NULL;
    if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(gate_bias, 4) || !aligned(logits, 4) ||
        !aligned(topk_idx, 4) || !aligned(topk_w, 4) || !aligned(group_offsets, 4) ||
        !aligned(sorted_token, 4) || !aligned(row_of_slot, 4))
        return MOE_ERR_ALIGN;
    switch (desc->hidden / 512) {
        case 1: launch_small<1>(desc, T, x, w_router, gate_bias, logits, topk_idx, topk_w, group_offsets, sorted_token, row_of_slot, sync, st); break;
        case 2: launch_small<2>(desc, T, x, w_router, gate_bias, logits, topk_idx, topk_w, group_offsets, sorted_token, row_of_slot, sync, st); break;
        case 4: launch_small<4>(desc, T, x, w_router, gate_bias, logits, topk_idx, topk_w, group_offsets, sorted_token, row_of_slot, sync, st); break;
        case 8: launch_small<8>(desc, T, x, w_router, gate_bias, logits, topk_idx, topk_w, group_offsets, sorted_token, row_of_slot, sync, st); break;
        default: return MOE_ERR_UNSUPPORTED;
    }
    return launch_status();
}

}  // namespace moe

extern "C" moe_status moe_route_permute(const moe_layer_desc *desc, int32_t T, const uint16_t *x,
                                        const uint16_t *w_router, const float *gate_bias,
                                        float *logits, int32_t *topk_idx, float *topk_w,
                                        int32_t *group_offsets, int32_t *sorted_token,
                                        int32_t *row_of_slot, void *ws, size_t ws_bytes, void *stream) {
    MOE_TRY(check_desc(desc));
    MOE_TRY(check_tokens(T));
    if (T == 0) return MOE_OK;
    MOE_TRY(check_workspace(desc, T, ws, ws_bytes));
    return route_permute(desc, T, x, w_router, gate_bias, logits, topk_idx, topk_w, group_offsets,
                         sorted_token, row_of_slot, ws, (hipStream_t)stream);
}

// ---------------------------------------------------------------- no allocation
// moe_route_permute_noalloc: the workspace of moe_route_permute in the
// library's own device memory, for callers that cannot allocate.  `scratch`
// below is the host-side name of that array: its device address comes from
// hipGetSymbolAddress, once per device (each GPU holds its own copy), and only
// that address is ever handed to a kernel.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_WS_BYTES];

namespace moe {
namespace {

static_assert(kWsHeaderBytes + (MOE_NOALLOC_MAX_TOKENS + 1023) / 1024 * 320 * sizeof(int32_t) <=
                  MOE_NOALLOC_WS_BYTES,
              "the static scratch holds the workspace of MOE_NOALLOC_MAX_TOKENS tokens");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];

// zero the header (the small-batch arrival counter starts at zero; the rest
// of the scratch is rewritten by every call): plain vector stores
__global__ void k_clear_header(uint32_t *h) {
    if (threadIdx.x < kWsHeaderBytes / 4) h[threadIdx.x] = 0u;
}

// The current device's scratch address; on its first use on a device the
// header is cleared on `st` (ahead of the call's own work).
moe_status noalloc_scratch(hipStream_t st, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_DEVICE;
        hipLaunchKernelGGL(k_clear_header, dim3(1), dim3(64), 0, st, (uint32_t *)p);
        MOE_TRY(launch_status());
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_route_permute_noalloc(const moe_layer_desc *desc, int32_t T, const uint16_t *x,
                                                const uint16_t *w_router, const float *gate_bias,
                                                float *logits, int32_t *topk_idx, float *topk_w,
                                                int32_t *group_offsets, int32_t *sorted_token,
                                                int32_t *row_of_slot, void *stream) {
    MOE_TRY(check_desc(desc));
    MOE_TRY(check_tokens(T));
    if (T == 0) return MOE_OK;
    if (T > MOE_NOALLOC_MAX_TOKENS) return MOE_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    void *ws = nullptr;
    MOE_TRY(noalloc_scratch(st, &ws));
    return route_permute(desc, T, x, w_router, gate_bias, logits, topk_idx, topk_w, group_offsets,
                         sorted_token, row_of_slot, ws, st);
}
