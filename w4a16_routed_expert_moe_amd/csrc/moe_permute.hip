// moe_permute.hip -- token permutation by expert on gfx950.
//
// The expert GEMM reads its rows through an index list (the "indexed" MoE
// GEMM of "Throughputmaxxing: DeepSeek-V4-Flash on Isambard-AI", "A pass through
// the model").  The slots (t, j) are counting-sorted by group, stable in
// flat slot order; the shared expert is the last group and receives every
// token in order.
//
// One workgroup does the whole sort (it is a few microseconds of work even
// at 8192 tokens, and one launch is what matters at decode):
//   1. per-group counts with LDS atomics (order-free, so deterministic);
//   2. one wave scans the counts into group_offsets;
//   3. tokens are taken in chunks of 1024: each token sets its bit in a
//      per-group 1024-bit LDS mask; the rank of slot (t, j) in its group is
//      the running base of the group plus the number of set bits below t,
//      which is exactly the stable order; the bases then advance by the
//      chunk's counts.
// A token picks each routed expert at most once, so one bit per (group,
// token) suffices.
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
    __shared__ int count[kMaxGroups];
    __shared__ int base[kMaxGroups];
    __shared__ unsigned long long mask[kMaxGroups][kWords];
    const int tid = threadIdx.x;
    const int G = E + ns, S = k + ns;

    for (int g = tid; g < G; g += kChunk) count[g] = 0;
    __syncthreads();
    for (int t = tid; t < T; t += kChunk)
        for (int j = 0; j < k; ++j) {
            int g = topk_idx[(size_t)t * k + j];
            g = min(max(g, 0), E - 1);
            atomicAdd(&count[g], 1);
        }
    if (tid == 0 && ns) count[E] = T;
    __syncthreads();

    if (tid < kWave) {  // exclusive scan: lane l owns groups 5l..5l+4
        const int l = tid;
        int local[5];
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int g = 5 * l + i;
            local[i] = g < G ? count[g] : 0;
            sum += local[i];
        }
        int run = wave_incl_scan(sum) - sum;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int g = 5 * l + i;
            if (g < G) {
                base[g] = run;
                offsets[g] = run;
            }
            run += local[i];
        }
        if (l == kWave - 1) offsets[G] = run;
    }
    __syncthreads();
    const int shared_base = ns ? base[E] : 0;

    for (int c0 = 0; c0 < T; c0 += kChunk) {
        for (int i = tid; i < G * kWords; i += kChunk) (&mask[0][0])[i] = 0ull;
        __syncthreads();
        const int t = c0 + tid;
        const int w = tid >> 6;
        const unsigned long long bit = 1ull << (tid & 63);
        int gs[8];
        if (t < T) {
            for (int j = 0; j < k; ++j) {
                int g = topk_idx[(size_t)t * k + j];
                g = min(max(g, 0), E - 1);
                gs[j] = g;
                atomicOr(&mask[g][w], bit);
            }
        }
        __syncthreads();
        if (t < T) {
            for (int j = 0; j < k; ++j) {
                const int g = gs[j];
                int rank = __popcll(mask[g][w] & (bit - 1));
                for (int q = 0; q < w; ++q) rank += __popcll(mask[g][q]);
                const int pos = base[g] + rank;
                sorted_token[pos] = t;
                row_of_slot[(size_t)t * S + j] = pos;
            }
            if (ns) {
                const int pos = shared_base + t;
                sorted_token[pos] = t;
                row_of_slot[(size_t)t * S + k] = pos;
            }
        }
        __syncthreads();
        for (int g = tid; g < E; g += kChunk) {
            int n = 0;
            for (int q = 0; q < kWords; ++q) n += __popcll(mask[g][q]);
            base[g] += n;
        }
        __syncthreads();
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
    hipLaunchKernelGGL(k_permute, dim3(1), dim3(kChunk), 0, (hipStream_t)stream, topk_idx, T,
                       desc->n_routed, desc->top_k, desc->n_shared, group_offsets, sorted_token,
                       row_of_slot);
    return launch_status();
}
