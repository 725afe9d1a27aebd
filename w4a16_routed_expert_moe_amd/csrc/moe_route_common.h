// moe_route_common.h -- the routing arithmetic shared by every kernel that
// routes tokens (moe_route.hip, and the single-launch decode step in
// moe_decode.hip), so that all of them choose the same experts to the last
// bit.  The definition (header of moe_route.hip and the ABI header): fp32
// logits in a fixed summation order, the library's own fp32 exp for the
// sigmoid, key = score + fp32 gate bias, top-k with ties to the lower
// index, weights renormalised in slot order.
#pragma once

#include "moe_common.h"

// No multiply-add contraction anywhere after this point: the routing sums are
// fixed to the operation, and the kernels that include this file write every
// fused multiply-add they want explicitly.
#pragma clang fp contract(off)

namespace moe {
namespace route {

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

// One router logit, in the order above: lane l holds the eight bf16
// elements 512j + 8l + u of x and of the router row (one 16-byte word per
// j), accumulates them with fused multiply-adds (j, then u, ascending), and
// the wave adds its 64 partials by the tree.  Every lane returns the sum.
template <int HJ>
__device__ __forceinline__ float router_dot(const u32x4 (&xv)[HJ], const u32x4 (&wv)[HJ]) {
    float P = 0.0f;
#pragma unroll
    for (int j = 0; j < HJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            P = __builtin_fmaf(bf16lo_to_f32(xv[j][q]), bf16lo_to_f32(wv[j][q]), P);
            P = __builtin_fmaf(bf16hi_to_f32(xv[j][q]), bf16hi_to_f32(wv[j][q]), P);
        }
    return wave_tree_sum(P);
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

// The wave-wide maximum of one 32-bit word per lane (every lane receives
// it).  The partner of a lane at each level only has to lie in the other
// half of the group being combined: quad permutes for groups of 2 and 4,
// row_half_mirror and row_mirror for 8 and 16 (DPP), and a swap of rows /
// halves of the wave for 32 and 64.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint32_t wave_max32(uint32_t v) {
    v = umax32(v, dpp32<0xB1>(v));   // quad_perm 1,0,3,2
    v = umax32(v, dpp32<0x4E>(v));   // quad_perm 2,3,0,1
    v = umax32(v, dpp32<0x141>(v));  // row_half_mirror
    v = umax32(v, dpp32<0x140>(v));  // row_mirror
    {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        v = umax32((uint32_t)r[0], (uint32_t)r[1]);
    }
    {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        v = umax32((uint32_t)r[0], (uint32_t)r[1]);
    }
    return v;
}

__device__ __forceinline__ float readlane_f32(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// One wave selects for one token from its scores s = sigmoid(logit) and gate
// biases, held four per lane: lane l has experts 4l..4l+3 in sc[0..3] and
// bs[0..3] (entries past E are ignored).  Each lane sorts its four packed
// keys.  Then k rounds each take the wave-wide maximum of the lanes' leading
// keys' upper halves (the score key); of the lanes that hold it, the lowest
// has the lowest expert index (lane l holds experts 4l..4l+3, and a lane's
// equal keys are sorted by index), so it holds the round's key under the
// order "larger key, then lower index", and moves on to its next key.
// Round j's expert goes to lane j, so lanes j < k end with the k largest
// keys in descending order (select_experts); the weights are renormalised in
// that order (route_weights).
__device__ __forceinline__ int select_experts(const float (&sc)[4], const float (&bs)[4], int E, int k) {
    const int l = lane_id();
    uint64_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = 4 * l + i;
        v[i] = 0;  // below every real key
        if (e < E) v[i] = pack_key(sc[i] + bs[i], e);
    }
    ce_desc(v[0], v[1]);
    ce_desc(v[2], v[3]);
    ce_desc(v[0], v[2]);
    ce_desc(v[1], v[3]);
    ce_desc(v[1], v[2]);
    uint32_t kh[4], kl[4];  // score key, 0xFFFFFFFF - expert
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        kh[i] = (uint32_t)(v[i] >> 32);
        kl[i] = (uint32_t)v[i];
    }

    int e_sel = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // k <= 8
        if (j >= k) break;
        const uint32_t best = wave_max32(kh[0]);
        // k <= E: some lane's head is a real key, so the mask is not empty
        const int w = __builtin_ctzll(__ballot(kh[0] == best));
        const uint32_t code = (uint32_t)__builtin_amdgcn_readlane((int)kl[0], w);
        if (l == j) e_sel = (int)(0xFFFFFFFFu - code);
        if (l == w) {
            kh[0] = kh[1];
            kh[1] = kh[2];
            kh[2] = kh[3];
            kh[3] = 0;
            kl[0] = kl[1];
            kl[1] = kl[2];
            kl[2] = kl[3];
        }
    }
    return e_sel;
}

// The routing weights of the chosen experts (lane j < k holds the j-th,
// e_sel from select_experts): each chosen score over their sum in slot
// order, times routed_scale; lanes j < k write idx_out[j] and w_out[j].
__device__ __forceinline__ void route_weights(const float (&sc)[4], int e_sel, int k, float routed_scale,
                                              int32_t *__restrict__ idx_out, float *__restrict__ w_out) {
    const int l = lane_id();
    // the chosen expert's score, from the lane that holds it
    const int src = min(max(e_sel, 0), 255) >> 2, part = e_sel & 3;
    const float s0 = __shfl(sc[0], src, kWave), s1 = __shfl(sc[1], src, kWave);
    const float s2 = __shfl(sc[2], src, kWave), s3 = __shfl(sc[3], src, kWave);
    const float s_sel = part == 0 ? s0 : part == 1 ? s1 : part == 2 ? s2 : s3;
    float S = readlane_f32(s_sel, 0);  // slot order
#pragma unroll
    for (int j = 1; j < 8; ++j)
        if (j < k) S = S + readlane_f32(s_sel, j);
    if (l < k) {
        idx_out[l] = e_sel;
        w_out[l] = __fdiv_rn(s_sel, S) * routed_scale;
    }
}

__device__ __forceinline__ int select_scores(const float (&sc)[4], const float (&bs)[4], int E, int k,
                                             float routed_scale, int32_t *__restrict__ idx_out,
                                             float *__restrict__ w_out) {
    const int e_sel = select_experts(sc, bs, E, k);
    route_weights(sc, e_sel, k, routed_scale, idx_out, w_out);
    return e_sel;
}

// The same from logits lg[0..E) (any memory the wave can read).
__device__ __forceinline__ int select_token(const float *__restrict__ lg,
                                            const float *__restrict__ bias, int E, int k,
                                            float routed_scale, int32_t *__restrict__ idx_out,
                                            float *__restrict__ w_out) {
    const int l = lane_id();
    float sc[4], bs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = 4 * l + i;
        sc[i] = e < E ? sigmoid_f32(lg[e]) : 0.0f;
        bs[i] = e < E ? bias[e] : 0.0f;
    }
    return select_scores(sc, bs, E, k, routed_scale, idx_out, w_out);
}

// ------------------------------------------------------------------ permute
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

}  // namespace route
}  // namespace moe
