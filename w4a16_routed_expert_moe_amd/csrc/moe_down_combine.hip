// moe_down_combine.hip -- the down projection and the weighted combine in one
// launch, for decode batches (T <= 4) on gfx950.
//
// For one token the layer ends with out = y_shared + sum_j w_j y_j, where
// y_j = h_j . W2_{e_j}^T over the token's k routed experts e_j and the shared
// expert (model card "canada-quant/DeepSeek-V4-Flash-W4A16-FP8-MTP",
// "Architecture & precision"; the routing weights w_j as for moe_route).  The
// separate down GEMM and combine each pay a launch and a dependent load at
// bs = 1; here a workgroup owns 16 output columns, streams those 16 weight
// rows of every (token, slot) pair in turn -- the same INT4 stream as the
// grouped GEMM -- and adds w_j * y_j straight into its fp32 output, which it
// rounds to bf16 once.  y is never stored.
//
// Layout per workgroup: sixteen waves, four per K quarter (KGW 128-wide k
// groups each), the slots dealt round the four waves of a quarter; a wave
// loads two slots' weights, scales and h slices at a time.  The MFMA tile has 16
// rows of which only row 0 (the slot's h row) is used: lanes 0..15 of each
// quarter read h through LDS, the others feed zeros.
#include <type_traits>

#include "moe_gemm_common.h"

namespace moe {
namespace {

constexpr int kMaxTok = 4;

// 16 waves: four K quarters x four slot groups (slot f goes to group f % 4);
// a wave keeps two slots' loads in flight at a time.  Sixteen waves a CU keep
// enough loads in flight to stream at full rate (four waves did not).
constexpr int kSlotGroups = 4;
constexpr int kSlotChunk = 2;

template <int KGW>
__global__ __launch_bounds__(256 * kSlotGroups) void k_down_combine(
    const uint16_t *__restrict__ h, const u32x4 *__restrict__ wq, const uint16_t *__restrict__ scales,
    const int32_t *__restrict__ topk_idx, const float *__restrict__ topk_w,
    const int32_t *__restrict__ row_of_slot, int T, int E, int k, int ns, int N, int K, int R,
    uint16_t *__restrict__ out) {
    const int wave = threadIdx.x >> 6, l = lane_id();
    const int m = l & 15, q = l >> 4;
    const int kq = wave & 3, sgrp = wave >> 2;  // K quarter, slot group
    const int nt = blockIdx.x;  // output columns 16*nt .. 16*nt+15
    const int KG = K >> 7, NT = N >> 4;
    const int kg0 = kq * KGW;
    const int S = k + ns, nslots = T * S;
    const int G = E + ns;
    // this wave's slots: sgrp, sgrp + 4, ...
    const int nmine = nslots > sgrp ? (nslots - sgrp + kSlotGroups - 1) / kSlotGroups : 0;

    // the wave's k slice of the h rows of the current chunk; slot i of the
    // chunk at [i][KGW*128], plus one zero row for lanes m != 0
    constexpr int kSlice = KGW * 128;
    __shared__ __attribute__((aligned(16))) uint16_t hs[4 * kSlotGroups][kSlotChunk][kSlice];
    __shared__ float red[4 * kSlotGroups][kMaxTok][16];

    auto slot_info = [&](int f, int &g, int &r, float &w) {
        const int t = f / S, j = f - t * S;
        if (j < k) {
            g = topk_idx[t * k + j];
            w = topk_w[t * k + j];
        } else {
            g = E;
            w = 1.0f;
        }
        g = min(max(g, 0), G - 1);  // ids come from moe_route; keep every read in bounds
        r = min(max(row_of_slot[f], 0), R - 1);
    };

    constexpr int kHv = kSlice >= 512 ? kSlice / 512 : 1;  // 16-byte pieces of h per lane
    u32x4 wv[kSlotChunk][KGW];
    uint16_t sraw[kSlotChunk][KGW];
    u32x4 hv[kSlotChunk][kHv];
    float wslot[kSlotChunk];
    int tslot[kSlotChunk];
    // registers of chunk c: weights, scales and the wave's slice of each h row
    auto issue = [&](int c) {
#pragma unroll
        for (int i = 0; i < kSlotChunk; ++i) {
            int g, r;
            float w;
            const int f = sgrp + kSlotGroups * min(c * kSlotChunk + i, nmine - 1);  // past the end: repeats
            slot_info(f, g, r, w);
            g = __builtin_amdgcn_readfirstlane(g);
            r = __builtin_amdgcn_readfirstlane(r);
            wslot[i] = w;
            tslot[i] = f / S;
            const u32x4 *wg = wq + ((size_t)(g * NT + nt) * KG + kg0) * kWave + l;
            const uint16_t *sg = scales + ((size_t)g * N + 16 * nt + m) * KG + kg0;
#pragma unroll
            for (int j = 0; j < KGW; ++j) {
                wv[i][j] = wg[(size_t)j * kWave];
                sraw[i][j] = sg[j];
            }
            // lanes past the slice (KGW < 4) re-read its start
            const int off = (8 * l) % kSlice;
#pragma unroll
            for (int c8 = 0; c8 < kHv; ++c8)
                hv[i][c8] = *(const u32x4 *)(h + (size_t)r * K + kg0 * 128 + 512 * c8 + off);
        }
    };
    auto stage_h = [&]() {  // the chunk's h slices into LDS (their loads must have landed)
#pragma unroll
        for (int i = 0; i < kSlotChunk; ++i)
#pragma unroll
            for (int c8 = 0; c8 < kHv; ++c8)
                if (512 * c8 + 8 * l < kSlice) *(u32x4 *)&hs[wave][i][512 * c8 + 8 * l] = hv[i][c8];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    bf16x8 bneg;
#pragma unroll
    for (int i = 0; i < 8; ++i) bneg[i] = __builtin_bit_cast(__bf16, kNeg136);
    f32x4 acc[kMaxTok];
#pragma unroll
    for (int t = 0; t < kMaxTok; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nchunks = (nmine + kSlotChunk - 1) / kSlotChunk;
    for (int c = 0; c < nchunks; ++c) {
        issue(c);
        stage_h();
#pragma unroll
        for (int i = 0; i < kSlotChunk; ++i) {
            if (c * kSlotChunk + i >= nmine) break;  // wave-uniform
            f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KGW; ++j) {
                u32x4 av[4];
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    av[d] = *(const u32x4 *)&hs[wave][i][j * 128 + 32 * q + 8 * d];
                    if (m != 0) av[d] = u32x4{0u, 0u, 0u, 0u};
                }
                f32x4 tt = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int d = 0; d < 4; ++d) tt = mfma16(__builtin_bit_cast(bf16x8, av[d]), bneg, tt);
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    tt = mfma16(__builtin_bit_cast(bf16x8, av[d]), unpack_codes(wv[i][j][d]), tt);
                const float sc = half_bits_to_f32(sraw[i][j]);
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = __builtin_fmaf(sc, tt[e], y[e]);
            }
            const float w = wslot[i];
            const int t = tslot[i];
#pragma unroll
            for (int tk = 0; tk < kMaxTok; ++tk)
                if (tk == t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[tk][e] = __builtin_fmaf(w, y[e], acc[tk][e]);
        }
        // every lane is done reading this chunk's h before the next one lands
        __builtin_amdgcn_wave_barrier();
    }

    // add the four waves' k partials; lanes 0..15 hold row 0 = the token's
    // output for column 16*nt + lane
    if (l < 16)
#pragma unroll
        for (int tk = 0; tk < kMaxTok; ++tk) red[wave][tk][l] = acc[tk][0];
    __syncthreads();
    if (wave == 0 && l < 16) {
        for (int tk = 0; tk < T; ++tk) {
            float v = red[0][tk][l];
            for (int w2 = 1; w2 < 4 * kSlotGroups; ++w2) v += red[w2][tk][l];
            out[(size_t)tk * N + 16 * nt + l] = f32_to_bf16(v);
        }
    }
}

template <int KGW>
void launch_down_combine(const uint16_t *h, const u32x4 *wq, const uint16_t *scales,
                         const int32_t *topk_idx, const float *topk_w, const int32_t *row_of_slot,
                         int T, int E, int k, int ns, int N, int K, int R, uint16_t *out,
                         hipStream_t st) {
    hipLaunchKernelGGL((k_down_combine<KGW>), dim3(N / 16), dim3(256 * kSlotGroups), 0, st, h, wq, scales, topk_idx,
                       topk_w, row_of_slot, T, E, k, ns, N, K, R, out);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_w4a16_down_combine(const moe_layer_desc *desc, int32_t T, const uint16_t *h,
                                             const uint8_t *w_packed, const uint16_t *w_scales,
                                             const int32_t *topk_idx, const float *topk_w,
                                             const int32_t *row_of_slot, uint16_t *out,
                                             void *stream) {
    MOE_TRY(check_desc(desc));
    MOE_TRY(check_tokens(T));
    if (T > MOE_DOWN_COMBINE_MAX_TOKENS) return MOE_ERR_UNSUPPORTED;
    const int H = desc->hidden, I = desc->inter, KG = I / 128;
    if (KG != 4 && KG != 8 && KG != 16 && KG != 32) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!h || !w_packed || !w_scales || !topk_idx || !topk_w || !row_of_slot || !out)
        return MOE_ERR_NULL;
    if (!aligned(h, 16) || !aligned(w_packed, 16) || !aligned(w_scales, 2) || !aligned(topk_idx, 4) ||
        !aligned(topk_w, 4) || !aligned(row_of_slot, 4) || !aligned(out, 2))
        return MOE_ERR_ALIGN;
    const int E = desc->n_routed, k = desc->top_k, ns = desc->n_shared;
    const int R = T * (k + ns);
    hipStream_t st = (hipStream_t)stream;
    const u32x4 *wq = (const u32x4 *)w_packed;
    switch (KG / 4) {
        case 1: launch_down_combine<1>(h, wq, w_scales, topk_idx, topk_w, row_of_slot, T, E, k, ns, H, I, R, out, st); break;
        case 2: launch_down_combine<2>(h, wq, w_scales, topk_idx, topk_w, row_of_slot, T, E, k, ns, H, I, R, out, st); break;
        case 4: launch_down_combine<4>(h, wq, w_scales, topk_idx, topk_w, row_of_slot, T, E, k, ns, H, I, R, out, st); break;
        default: launch_down_combine<8>(h, wq, w_scales, topk_idx, topk_w, row_of_slot, T, E, k, ns, H, I, R, out, st); break;
    }
    return launch_status();
}
