// moe_permute.hip -- token permutation by expert on gfx950.
//
// The expert GEMM reads its rows through an index list (the "indexed" MoE
// GEMM of "Throughputmaxxing: DeepSeek-V4-Flash on Isambard-AI", "A pass through
// the model").  The slots (t, j) are counting-sorted by group, stable in
// flat slot order; the shared expert is the last group and receives every
// token in order.
//
// Tokens come in chunks of 1024, one workgroup each.  Up to one chunk the
// sort is one launch (k_permute_one): count, scan, rank.  Past one chunk it
// is three launches through the caller's workspace, each linear in T:
//   1. k_permute_count: each chunk's slots per group (LDS atomics,
//      order-free, so deterministic) into counts[chunk][group];
//   2. k_permute_scan: one workgroup turns the counts into each chunk's
//      base row per group (the group's offset plus the slots of the chunks
//      before) and writes the group offsets;
//   3. k_permute_scatter: each token of the chunk sets its bit in a
//      per-group 1024-bit LDS mask; the rank of slot (t, j) in its group is
//      the chunk's base plus the number of set bits below t (a per-word
//      prefix of the set bits, then one popcount), which is exactly the
//      stable order.
// A token picks each routed expert at most once, so one bit per (group,
// token) suffices.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kMaxGroups = 257;
constexpr int kChunk = 1024;
constexpr int kWords = kChunk / 64;

constexpr int kGP = 320;  // row stride of the per-chunk table in the workspace (>= kMaxGroups)

// Slots of the chunk's tokens per group, into LDS cnt[0..G) (zeroed here).
__device__ __forceinline__ void count_chunk(const int32_t *__restrict__ topk_idx, int T, int E, int k,
                                            int ns, int c0, int *cnt) {
    const int tid = threadIdx.x, G = E + ns;
    for (int g = tid; g < G; g += kChunk) cnt[g] = 0;
    __syncthreads();
    const int n = min(T - c0, kChunk) * k;  // flat slots (t - c0)*k + j of the chunk
    const int32_t *ids = topk_idx + (size_t)c0 * k;
    for (int i0 = tid; i0 < n; i0 += 4 * kChunk) {
        int gv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * kChunk;
            gv[u] = i < n ? min(max(ids[i], 0), E - 1) : -1;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (gv[u] >= 0) atomicAdd(&cnt[gv[u]], 1);
    }
    if (tid == 0 && ns) cnt[E] = min(T - c0, kChunk);
    __syncthreads();
}

// Exclusive scan of cnt[0..G) by one wave (lane l owns groups 5l..5l+4):
// base[g] = add[g] + (slots of the groups before g); offsets written when
// given.
__device__ __forceinline__ void scan_groups(const int *cnt, const int *add, int G, int *base,
                                            int32_t *__restrict__ offsets) {
    const int l = threadIdx.x;
    int local[5];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int g = 5 * l + i;
        local[i] = g < G ? cnt[g] : 0;
        sum += local[i];
    }
    int run = wave_incl_scan(sum) - sum;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int g = 5 * l + i;
        if (g < G) {
            base[g] = run + (add ? add[g] : 0);
            if (offsets) offsets[g] = run;
        }
        run += local[i];
    }
    if (offsets && l == kWave - 1) offsets[G] = run;
}

// Stable ranks inside the chunk from per-group token masks; base[g] is the
// chunk's first row of group g.
__device__ __forceinline__ void scatter_chunk(const int32_t *__restrict__ topk_idx, int T, int E, int k,
                                              int ns, int c0, const int *base,
                                              unsigned long long (*mask)[kWords], int (*wpre)[kWords],
                                              int32_t *__restrict__ sorted_token,
                                              int32_t *__restrict__ row_of_slot) {
    const int tid = threadIdx.x, G = E + ns, S = k + ns;
    for (int i = tid; i < G * kWords; i += kChunk) (&mask[0][0])[i] = 0ull;
    __syncthreads();
    const int t = c0 + tid;
    const int w = tid >> 6;
    const unsigned long long bit = 1ull << (tid & 63);
    int gs[8];
    if (t < T) {
        for (int j = 0; j < k; ++j) {
            const int g = min(max(topk_idx[(size_t)t * k + j], 0), E - 1);
            gs[j] = g;
            atomicOr(&mask[g][w], bit);
        }
    }
    __syncthreads();
    for (int g = tid; g < G; g += kChunk) {
        int run = 0;
#pragma unroll
        for (int q = 0; q < kWords; ++q) {
            wpre[g][q] = run;
            run += __popcll(mask[g][q]);
        }
    }
    __syncthreads();
    if (t < T) {
        for (int j = 0; j < k; ++j) {
            const int g = gs[j];
            const int rank = wpre[g][w] + __popcll(mask[g][w] & (bit - 1));
            const int pos = base[g] + rank;
            sorted_token[pos] = t;
            row_of_slot[(size_t)t * S + j] = pos;
        }
        if (ns) {
            const int pos = base[E] + tid;
            sorted_token[pos] = t;
            row_of_slot[(size_t)t * S + k] = pos;
        }
    }
}

// T <= 1024: the whole sort in one workgroup.
__global__ __launch_bounds__(1024) void k_permute_one(const int32_t *__restrict__ topk_idx, int T,
                                                      int E, int k, int ns,
                                                      int32_t *__restrict__ offsets,
                                                      int32_t *__restrict__ sorted_token,
                                                      int32_t *__restrict__ row_of_slot) {
    __shared__ int cnt[kMaxGroups];
    __shared__ int base[kMaxGroups];
    __shared__ unsigned long long mask[kMaxGroups][kWords];
    __shared__ int wpre[kMaxGroups][kWords];  // set bits of a group's mask in the words below
    count_chunk(topk_idx, T, E, k, ns, 0, cnt);
    if (threadIdx.x < kWave) scan_groups(cnt, nullptr, E + ns, base, offsets);
    scatter_chunk(topk_idx, T, E, k, ns, 0, base, mask, wpre, sorted_token, row_of_slot);
}

// T > 1024, pass 1: counts[chunk][g] in the workspace.
__global__ __launch_bounds__(1024) void k_permute_count(const int32_t *__restrict__ topk_idx, int T,
                                                        int E, int k, int ns,
                                                        int32_t *__restrict__ counts) {
    __shared__ int cnt[kMaxGroups];
    count_chunk(topk_idx, T, E, k, ns, blockIdx.x * kChunk, cnt);
    for (int g = threadIdx.x; g < E + ns; g += kChunk) counts[(size_t)blockIdx.x * kGP + g] = cnt[g];
}

// T > 1024, pass 2 (one workgroup): thread g walks group g's column of the
// table, replacing each count by the slots of that group in the chunks
// before (loads eight chunks ahead); then one wave scans the group totals
// into the offsets, and each chunk's entry gets its group's offset added.
__global__ __launch_bounds__(1024) void k_permute_scan(int nchunks, int G, int32_t *__restrict__ counts,
                                                       int32_t *__restrict__ offsets) {
    __shared__ int total[kMaxGroups];
    __shared__ int goff[kMaxGroups];
    const int g = threadIdx.x;
    if (g < G) {
        int run = 0;
        int c = 0;
        for (; c + 8 <= nchunks; c += 8) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = counts[(size_t)(c + u) * kGP + g];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                counts[(size_t)(c + u) * kGP + g] = run;
                run += v[u];
            }
        }
        for (; c < nchunks; ++c) {
            const int v = counts[(size_t)c * kGP + g];
            counts[(size_t)c * kGP + g] = run;
            run += v;
        }
        total[g] = run;
    }
    __syncthreads();
    if (threadIdx.x < kWave) scan_groups(total, nullptr, G, goff, offsets);
    __syncthreads();
    if (g < G) {
        const int o = goff[g];
        for (int c2 = 0; c2 < nchunks; ++c2) counts[(size_t)c2 * kGP + g] += o;
    }
}

// T > 1024, pass 3: each chunk's stable ranks from its row of bases.
__global__ __launch_bounds__(1024) void k_permute_scatter(const int32_t *__restrict__ topk_idx, int T,
                                                          int E, int k, int ns,
                                                          const int32_t *__restrict__ bases,
                                                          int32_t *__restrict__ sorted_token,
                                                          int32_t *__restrict__ row_of_slot) {
    __shared__ int base[kMaxGroups];
    __shared__ unsigned long long mask[kMaxGroups][kWords];
    __shared__ int wpre[kMaxGroups][kWords];
    for (int g = threadIdx.x; g < E + ns; g += kChunk) base[g] = bases[(size_t)blockIdx.x * kGP + g];
    scatter_chunk(topk_idx, T, E, k, ns, blockIdx.x * kChunk, base, mask, wpre, sorted_token, row_of_slot);
}

}  // namespace


size_t workspace_bytes(const moe_layer_desc *desc, int32_t T) {
    if (check_desc(desc) != MOE_OK || check_tokens(T) != MOE_OK) return 0;
    const size_t chunks = T > kChunk ? (size_t)((T + kChunk - 1) / kChunk) : 0;
    return kWsHeaderBytes + chunks * kGP * sizeof(int32_t);
}

moe_status check_workspace(const moe_layer_desc *desc, int32_t T, const void *ws, size_t ws_bytes) {
    if (!ws) return MOE_ERR_NULL;
    if (!aligned(ws, 16)) return MOE_ERR_ALIGN;
    if (ws_bytes < workspace_bytes(desc, T)) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

moe_status launch_permute(const moe_layer_desc *desc, int32_t T, const int32_t *topk_idx,
                          int32_t *group_offsets, int32_t *sorted_token, int32_t *row_of_slot,
                          void *ws, hipStream_t st) {
    const int E = desc->n_routed, k = desc->top_k, ns = desc->n_shared;
    if (T <= kChunk) {
        hipLaunchKernelGGL(k_permute_one, dim3(1), dim3(kChunk), 0, st, topk_idx, T, E, k, ns,
                           group_offsets, sorted_token, row_of_slot);
        return launch_status();
    }
    const int nchunks = (T + kChunk - 1) / kChunk;
    int32_t *counts = (int32_t *)((char *)ws + kWsHeaderBytes);
    hipLaunchKernelGGL(k_permute_count, dim3(nchunks), dim3(kChunk), 0, st, topk_idx, T, E, k, ns, counts);
    MOE_TRY(launch_status());
    hipLaunchKernelGGL(k_permute_scan, dim3(1), dim3(kChunk), 0, st, nchunks, E + ns, counts, group_offsets);
    MOE_TRY(launch_status());
    hipLaunchKernelGGL(k_permute_scatter, dim3(nchunks), dim3(kChunk), 0, st, topk_idx, T, E, k, ns, counts,
                       sorted_token, row_of_slot);
    return launch_status();
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_workspace_bytes(const moe_layer_desc *desc, int32_t T) {
    return workspace_bytes(desc, T);
}

extern "C" moe_status moe_permute(const moe_layer_desc *desc, int32_t T, const int32_t *topk_idx,
                                  int32_t *group_offsets, int32_t *sorted_token,
                                  int32_t *row_of_slot, void *ws, size_t ws_bytes, void *stream) {
    MOE_TRY(check_desc(desc));
    MOE_TRY(check_tokens(T));
    if (T == 0) return MOE_OK;
    if (!topk_idx || !group_offsets || !sorted_token || !row_of_slot) return MOE_ERR_NULL;
    if (!aligned(topk_idx, 4) || !aligned(group_offsets, 4) || !aligned(sorted_token, 4) ||
        !aligned(row_of_slot, 4))
        return MOE_ERR_ALIGN;
    if (T > kChunk) MOE_TRY(check_workspace(desc, T, ws, ws_bytes));
    return launch_permute(desc, T, topk_idx, group_offsets, sorted_token, row_of_slot, ws,
                          (hipStream_t)stream);
}
