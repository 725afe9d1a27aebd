// moe_layout.hip -- weight layout conversion, device-side synthetic weights,
// and the small ABI helpers.
//
// Prepack: canonical INT4 rows (two codes per byte, element 2c in the low
// nibble) -> the streamed layout of the grouped GEMM: 1 KB per (group,
// 16-row tile, 128-wide k group), lane l's 16 bytes covering row l%16 and
// k = 32*(l/16) + [0,32) of the k group, each 32-bit word holding its even
// elements in the low half-word and its odd elements in the high half-word,
// codes stored as q+8.  The conversion is a permutation of nibbles plus an
// XOR with 8, so it is bijective.  FP4 (E2M1) codes take the same 1 KB
// blocks with each 32-bit word copied as it is (eight consecutive elements,
// element j in bits [4j, 4j+4)): the hardware conversion reads them in that
// order.
//
// Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
// number generators", OOPSLA 2014) used in counter form, output i of the
// stream seeded with S being mix(S + (i+1)*gamma).
#include <cstring>

#include "moe_common.h"

namespace moe {
namespace {

template <bool FP4>
__global__ __launch_bounds__(256) void k_prepack(const uint32_t *__restrict__ src,
                                                 uint32_t *__restrict__ dst, int N, int K,
                                                 int64_t total_words) {
    const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= total_words) return;
    const int KG = K >> 7, NT = N >> 4;
    const int d = (int)(o & 3);
    const int l = (int)((o >> 2) & 63);
    int64_t rest = o >> 8;  // (g*NT + nt)*KG + kg
    const int kg = (int)(rest % KG);
    rest /= KG;
    const int nt = (int)(rest % NT);
    const int64_t g = rest / NT;
    const int n = nt * 16 + (l & 15);
    const int kbase = kg * 128 + 32 * (l >> 4) + 8 * d;
    const uint32_t cw = src[((g * N + n) * (int64_t)K + kbase) >> 3];  // 8 codes, k ascending
    if (FP4) {
        dst[o] = cw;
        return;
    }
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        w |= ((cw >> (8 * j)) & 0xFu) << (4 * j);             // element 2j
        w |= ((cw >> (8 * j + 4)) & 0xFu) << (16 + 4 * j);    // element 2j+1
    }
    dst[o] = w ^ 0x88888888u;
}

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t splitmix_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t tensor_stream_seed(uint64_t seed, int layer, int group, int kind) {
    const uint64_t tid = ((uint64_t)layer * 512u + (uint64_t)group) * 4u + (uint64_t)kind;
    return splitmix_mix(seed + (tid + 1u) * kGamma);
}

// one thread per 8-byte word of one group's canonical codes
__global__ __launch_bounds__(256) void k_gen_codes(uint64_t seed, int layer, int group0, int kind,
                                                   int64_t words_per_group, uint64_t *__restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int gi = blockIdx.y;
    if (i >= words_per_group) return;
    const uint64_t S = tensor_stream_seed(seed, layer, group0 + gi, kind);
    out[(int64_t)gi * words_per_group + i] = splitmix_mix(S + ((uint64_t)i + 1u) * kGamma);
}

__global__ __launch_bounds__(256) void k_gen_scales(uint64_t seed, int layer, int group0, int kind,
                                                    int64_t per_group, uint16_t *__restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int gi = blockIdx.y;
    if (i >= per_group) return;
    const uint64_t S = tensor_stream_seed(seed, layer, group0 + gi, kind);
    const uint64_t h = splitmix_mix(S + ((uint64_t)i + 1u) * kGamma);
    const float u = (float)(uint32_t)(h >> 40) * 0x1p-24f;   // exact: 24-bit integer
    float s = __builtin_fmaf(0.015f, u, 0.005f);
    // The definition rounds to fp32 first, then to fp16; keep the compiler from
    // fusing the two roundings into one mixed-precision fma.
    asm volatile("" : "+v"(s));
    out[(int64_t)gi * per_group + i] = __builtin_bit_cast(uint16_t, (_Float16)s);
}

// UE8M0 scale bytes: E = 120 + (h >> 62)
__global__ __launch_bounds__(256) void k_gen_ue8m0(uint64_t seed, int layer, int group0, int kind,
                                                   int64_t per_group, uint8_t *__restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int gi = blockIdx.y;
    if (i >= per_group) return;
    const uint64_t S = tensor_stream_seed(seed, layer, group0 + gi, kind);
    const uint64_t h = splitmix_mix(S + ((uint64_t)i + 1u) * kGamma);
    out[(int64_t)gi * per_group + i] = (uint8_t)(120u + (uint32_t)(h >> 62));
}

moe_status prepack(bool fp4, int32_t n_groups, int32_t N, int32_t K, const uint8_t *w_canonical,
                   uint8_t *w_packed, void *stream) {
    if (n_groups < 0 || N < 16 || N % 16 || K < 128 || K % 128 || N > 65536 || K > 65536)
        return MOE_ERR_SHAPE;
    if (n_groups == 0) return MOE_OK;
    if (!w_canonical || !w_packed) return MOE_ERR_NULL;
    if (!aligned(w_canonical, 4) || !aligned(w_packed, 16)) return MOE_ERR_ALIGN;
    const int64_t bytes = (int64_t)n_groups * N * K / 2;
    if ((const uint8_t *)w_canonical < w_packed + bytes && w_packed < (const uint8_t *)w_canonical + bytes)
        return MOE_ERR_SHAPE;  // overlapping buffers
    const int64_t words = bytes / 4;
    const int64_t blocks = (words + 255) / 256;
    if (blocks > 0x7FFFFFFF) return MOE_ERR_SHAPE;
    auto kern = fp4 ? k_prepack<true> : k_prepack<false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       (const uint32_t *)w_canonical, (uint32_t *)w_packed, N, K, words);
    return launch_status();
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_w4a16_prepack(int32_t n_groups, int32_t N, int32_t K,
                                        const uint8_t *w_canonical, uint8_t *w_packed,
                                        void *stream) {
    return prepack(false, n_groups, N, K, w_canonical, w_packed, stream);
}

extern "C" moe_status moe_mxfp4_prepack(int32_t n_groups, int32_t N, int32_t K,
                                        const uint8_t *w_canonical, uint8_t *w_packed,
                                        void *stream) {
    return prepack(true, n_groups, N, K, w_canonical, w_packed, stream);
}

extern "C" moe_status moe_gen_int4_codes(uint64_t seed, int32_t layer, int32_t group0,
                                         int32_t n_groups, int32_t kind, int32_t N, int32_t K,
                                         uint8_t *out, void *stream) {
    if (layer < 0 || group0 < 0 || n_groups < 0 || n_groups > 65535 || group0 + n_groups > 512 ||
        kind < 0 || kind > 3 || N < 1 || K < 16 || K % 16)
        return MOE_ERR_SHAPE;
    if (n_groups == 0) return MOE_OK;
    if (!out) return MOE_ERR_NULL;
    if (!aligned(out, 8)) return MOE_ERR_ALIGN;
    const int64_t words = (int64_t)N * K / 16;
    const int64_t bx = (words + 255) / 256;
    if (bx > 0x7FFFFFFF) return MOE_ERR_SHAPE;
    hipLaunchKernelGGL(k_gen_codes, dim3((unsigned)bx, n_groups), dim3(256), 0, (hipStream_t)stream,
                       seed, layer, group0, kind, words, (uint64_t *)out);
    return launch_status();
}

extern "C" moe_status moe_gen_fp16_scales(uint64_t seed, int32_t layer, int32_t group0,
                                          int32_t n_groups, int32_t kind, int32_t N, int32_t K,
                                          uint16_t *out, void *stream) {
    if (layer < 0 || group0 < 0 || n_groups < 0 || n_groups > 65535 || group0 + n_groups > 512 ||
        kind < 0 || kind > 3 || N < 1 || K < 128 || K % 128)
        return MOE_ERR_SHAPE;
    if (n_groups == 0) return MOE_OK;
    if (!out) return MOE_ERR_NULL;
    if (!aligned(out, 2)) return MOE_ERR_ALIGN;
    const int64_t per = (int64_t)N * (K / 128);
    const int64_t bx = (per + 255) / 256;
    if (bx > 0x7FFFFFFF) return MOE_ERR_SHAPE;
    hipLaunchKernelGGL(k_gen_scales, dim3((unsigned)bx, n_groups), dim3(256), 0, (hipStream_t)stream,
                       seed, layer, group0, kind, per, out);
    return launch_status();
}

extern "C" moe_status moe_gen_ue8m0_scales(uint64_t seed, int32_t layer, int32_t group0,
                                           int32_t n_groups, int32_t kind, int32_t N, int32_t K,
                                           uint8_t *out, void *stream) {
    if (layer < 0 || group0 < 0 || n_groups < 0 || n_groups > 65535 || group0 + n_groups > 512 ||
        kind < 0 || kind > 3 || N < 1 || K < 32 || K % 32)
        return MOE_ERR_SHAPE;
    if (n_groups == 0) return MOE_OK;
    if (!out) return MOE_ERR_NULL;
    const int64_t per = (int64_t)N * (K / 32);
    const int64_t bx = (per + 255) / 256;
    if (bx > 0x7FFFFFFF) return MOE_ERR_SHAPE;
    hipLaunchKernelGGL(k_gen_ue8m0, dim3((unsigned)bx, n_groups), dim3(256), 0, (hipStream_t)stream,
                       seed, layer, group0, kind, per, out);
    return launch_status();
}

extern "C" const char *moe_status_str(moe_status status) {
    // A C caller may pass any int: read the argument's bytes, not the C++
    // enum, whose valid values stop at its largest enumerator.
    int32_t s;
    static_assert(sizeof(s) == sizeof(status), "moe_status is 32-bit");
    memcpy(&s, &status, sizeof s);
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "null pointer argument";
        case MOE_ERR_SHAPE: return "size outside the supported limits";
        case MOE_ERR_UNSUPPORTED: return "unsupported mode";
        case MOE_ERR_ALIGN: return "misaligned pointer";
        case MOE_ERR_LAUNCH: return "kernel launch failed";
        case MOE_ERR_DEVICE: return "no usable gfx950 device";
        case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_bytes";
    }
    return "unknown status";
}

extern "C" int32_t moe_abi_version(void) { return MOE_W4A16_ABI_VERSION; }
