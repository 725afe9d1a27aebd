// moe_permute.hip -- token permutation by expert on gfx950.
//
// The expert GEMM reads its rows through an index list (the "indexed" MoE
// GEMM of "Throughputmaxxing: DeepSeek-V4-Flash on Isambard-AI", "A pass through
// the model").  The slots (t, j) are counting-sorted by group, stable in
// flat slot order; the shared expert is the last group and receives every
// token in order.
//
// One workgroup per chunk of 1024 tokens:
//   1. every workgroup counts the slots of all tokens per group with LDS
//      atomics (order-free, so deterministic), and separately those of the
//      tokens before its chunk -- a few hundred kilobytes from L2, read by
//      every workgroup (T*k slots each, T/1024 workgroups), instead of a pass
//      over the chunks one after another;
//   2. one wave scans the counts into the group offsets; a group's base for
//      the chunk is its offset plus the count before the chunk;
//   3. each token of the chunk sets its bit in a per-group 1024-bit LDS mask;
//      the rank of slot (t, j) in its group is the chunk's base plus the
//      number of set bits below t (a per-word prefix of the set bits, then
//      one popcount), which is exactly the stable order.
// A token picks each routed expert at most once, so one bit per (group,
// token) suffices.  At 8192 tokens this takes 24 us, and 13.6 us at 2048;
// one workgroup taking the chunks in turn took 141 and 36 us.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kMaxGroups = 257;
constexpr int kChunk = 1024;
constexpr int kWords = kChunk / 64;

__global__ __launch_bounds__(1024) void k_permute(const int32_t *__restrict__ topk_idx, int T,
                                                  int E, int k, int ns,
                                                  int32_t *__restrict__ offsets,
                                                  int32_t *__restrict__ sorted_token,
                                                  int32_t *__restrict__ row_of_slot) {
    __shared__ int before[kMaxGroups];  // slots per group, tokens before the chunk
    __shared__ int rest[kMaxGroups];    // slots per group, the chunk's tokens and later
    __shared__ int base[kMaxGroups];
    __shared__ unsigned long long mask[kMaxGroups][kWords];
    __shared__ int wpre[kMaxGroups][kWords];  // set bits of a group's mask in the words below
    const int tid = threadIdx.x;
    const int G = E + ns, S = k + ns;
    const int c0 = blockIdx.x * kChunk;  // first token of this workgroup's chunk

    for (int g = tid; g < G; g += kChunk) before[g] = rest[g] = 0;
    for (int i = tid; i < G * kWords; i += kChunk) (&mask[0][0])[i] = 0ull;
    __syncthreads();
    {
        // flat slot i = t*k + j, read coalesced, four per thread per pass
        const int n = T * k, nb = c0 * k;
        for (int i0 = tid; i0 < n; i0 += 4 * kChunk) {
            int gv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * kChunk;
                gv[u] = i < n ? min(max(topk_idx[i], 0), E - 1) : -1;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)  // one atomic per slot
                if (gv[u] >= 0) atomicAdd(i0 + u * kChunk < nb ? &before[gv[u]] : &rest[gv[u]], 1);
        }
    }
    if (tid == 0 && ns) {
        before[E] = c0;
        rest[E] = T - c0;
    }
    __syncthreads();

    if (tid < kWave) {  // exclusive scan: lane l owns groups 5l..5l+4
        const int l = tid;
        int local[5];
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int g = 5 * l + i;
            local[i] = g < G ? before[g] + rest[g] : 0;
            sum += local[i];
        }
        int run = wave_incl_scan(sum) - sum;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int g = 5 * l + i;
            if (g < G) {
                base[g] = run + before[g];
                if (blockIdx.x == 0) offsets[g] = run;
            }
            run += local[i];
        }
        if (l == kWave - 1 && blockIdx.x == 0) offsets[G] = run;
    }

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

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_permute(const moe_layer_desc *desc, int32_t T, const int32_t *topk_idx,
                                  int32_t *group_offsets, int32_t *sorted_token,
                                  int32_t *row_of_slot, void *stream) {
    MOE_TRY(check_desc(desc));
    MOE_TRY(check_tokens(T));
    if (T == 0) return MOE_OK;
    if (!topk_idx || !group_offsets || !sorted_token || !row_of_slot) return MOE_ERR_NULL;
    if (!aligned(topk_idx, 4) || !aligned(group_offsets, 4) || !aligned(sorted_token, 4) ||
        !aligned(row_of_slot, 4))
        return MOE_ERR_ALIGN;
    hipLaunchKernelGGL(k_permute, dim3((T + kChunk - 1) / kChunk), dim3(kChunk), 0, (hipStream_t)stream, topk_idx, T,
                       desc->n_routed, desc->top_k, desc->n_shared, group_offsets, sorted_token,
                       row_of_slot);
    return launch_status();
}
