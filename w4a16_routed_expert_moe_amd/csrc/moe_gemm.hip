// moe_gemm.hip -- grouped W4A16 GEMM of the expert projections on gfx950.
//
// Method: weight-only INT4 (one fp16 scale per 128 input elements, symmetric;
// model card "canada-quant/DeepSeek-V4-Flash-W4A16-FP8-MTP", "Component
// precisions"), dequantised in registers and multiplied with bf16
// activations on the matrix cores -- the scheme the Marlin kernel applies on
// Hopper ("Throughputmaxxing: DeepSeek-V4-Flash on Isambard-AI", "A pass through
// the model"), redesigned here for CDNA4.
//
// Weight-stream kernel (k_w4a16_stream).  One workgroup = 4 waves owns an
// n-block of 64 weight rows (for SwiGLU: 32 gate rows and the matching 32 up
// rows) and a chunk of <= 16 permuted rows of one group; the 4 waves split
// the K dimension and add their partial tiles through LDS at the end.
//   * B operand (weights): each lane reads 16 bytes of a 1 KB block of the
//     prepacked layout, so a wave load is one contiguous 1 KB stream; the
//     codes go straight from HBM to registers (no LDS).
//   * Unpack: a code u = q+8 placed under the bf16 exponent of 128 gives the
//     exact bf16 value 128+u with one AND-OR per pair of codes.  The MFMA
//     then yields sum A*(q+136); the -136*sum(A) term is one extra MFMA
//     chain per k group with a constant -136 B operand, shared by all
//     subtiles, and is fed in as the accumulator input.
//   * Scales: acc += s[n][kg] * tile after each 128-wide k group (fp32).
//   * A operand (activations): read from global through the row gather of the
//     permutation, 16 bytes per lane per MFMA, bf16 in natural k order.
// v_mfma_f32_16x16x32_bf16: A = 16 rows x 32 k (lane l: row l%16, k slots
// 8*(l/16)..+8), B = 32 k x 16 cols (lane l: col l%16), D = 16x16 fp32 with
// lane l holding rows 4*(l/16)..+4 of column l%16.  Here rows are permuted
// token rows and columns are weight rows.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kNSub = 4;          // 16-row weight subtiles per workgroup
constexpr int kRowsPerTile = 16;  // permuted rows per work item
constexpr uint32_t kMagic = 0x43004300u;  // bf16 128.0 in both halves
constexpr uint16_t kNeg136 = 0xC308;      // bf16 -136.0

__device__ __forceinline__ bf16x8 unpack_codes(uint32_t w) {
    u32x4 r;
    r[0] = (w & 0x000F000Fu) | kMagic;
    r[1] = ((w >> 4) & 0x000F000Fu) | kMagic;
    r[2] = ((w >> 8) & 0x000F000Fu) | kMagic;
    r[3] = ((w >> 12) & 0x000F000Fu) | kMagic;
    return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// Work item `tile` -> (group, first permuted row, row count).  Group g owns
// ceil(n_g / 16) consecutive work items.  Every wave computes it (no LDS).
__device__ __forceinline__ bool find_tile(int tile, const int32_t *__restrict__ offsets, int G,
                                          int &g_out, int &m0, int &mrows) {
    const int l = lane_id();
    int before = 0;
    for (int g0 = 0; g0 < G; g0 += kWave) {
        const int g = g0 + l;
        int n = 0, lo = 0;
        if (g < G) {
            lo = offsets[g];
            n = offsets[g + 1] - lo;
        }
        const int nt = (n + kRowsPerTile - 1) / kRowsPerTile;
        const int incl = wave_incl_scan(nt);
        const int total = __shfl(incl, kWave - 1, kWave);
        if (tile < before + total) {
            const bool mine = g < G && tile >= before + incl - nt && tile < before + incl;
            const uint64_t bal = __ballot(mine);
            const int src = __ffsll((unsigned long long)bal) - 1;
            const int chunk = tile - before - (__shfl(incl, src, kWave) - __shfl(nt, src, kWave));
            g_out = g0 + src;
            const int lo_s = __shfl(lo, src, kWave), n_s = __shfl(n, src, kWave);
            m0 = lo_s + chunk * kRowsPerTile;
            mrows = min(kRowsPerTile, n_s - chunk * kRowsPerTile);
            return true;
        }
        before += total;
    }
    return false;
}

template <int ACT>
__global__ __launch_bounds__(256) void k_w4a16_stream(
    const uint16_t *__restrict__ a, const int32_t *__restrict__ gather, int n_src,
    const u32x4 *__restrict__ wq, const uint16_t *__restrict__ scales,
    const int32_t *__restrict__ offsets, int G, int R, int N, int K, uint16_t *__restrict__ out,
    int NB) {
    __shared__ f32x4 red[4][kNSub][kWave];
    const int wave = threadIdx.x >> 6;
    const int l = lane_id();
    const int tile = blockIdx.x / NB;
    const int nb = blockIdx.x - tile * NB;
    int g, m0, mrows;
    if (!find_tile(tile, offsets, G, g, m0, mrows)) return;  // uniform over the block
    if (m0 < 0 || m0 >= R) return;                            // offsets not from moe_permute
    mrows = min(mrows, R - m0);

    const int KG = K >> 7, NT = N >> 4;
    const int kg0 = (wave * KG) >> 2, kg1 = ((wave + 1) * KG) >> 2;
    int nrow[kNSub];
#pragma unroll
    for (int s = 0; s < kNSub; ++s) {
        if (ACT == MOE_ACT_SWIGLU) {
            constexpr int half = kNSub / 2;
            const int c = nb * 16 * half + 16 * (s % half);
            nrow[s] = s < half ? c : (N >> 1) + c;
        } else {
            nrow[s] = nb * 16 * kNSub + 16 * s;
        }
    }

    const int m = l & 15, q = l >> 4;
    const uint16_t *arow = nullptr;
    if (m < mrows) {
        const int r = m0 + m;
        if (gather) {
            const int src = gather[r];
            if ((unsigned)src < (unsigned)n_src) arow = a + (size_t)src * K;
        } else {
            arow = a + (size_t)r * K;
        }
    }

    const u32x4 *wg = wq + (size_t)g * NT * KG * kWave;
    const uint16_t *sg = scales + (size_t)g * N * KG;
    bf16x8 bneg;
#pragma unroll
    for (int i = 0; i < 8; ++i) bneg[i] = __builtin_bit_cast(__bf16, kNeg136);

    f32x4 acc[kNSub];
#pragma unroll
    for (int s = 0; s < kNSub; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kg = kg0; kg < kg1; ++kg) {
        u32x4 av[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            av[d] = u32x4{0u, 0u, 0u, 0u};
            if (arow) av[d] = *(const u32x4 *)(arow + kg * 128 + 32 * q + 8 * d);
        }
        u32x4 wv[kNSub];
        float sc[kNSub];
#pragma unroll
        for (int s = 0; s < kNSub; ++s) {
            wv[s] = wg[((size_t)(nrow[s] >> 4) * KG + kg) * kWave + l];
            sc[s] = half_bits_to_f32(sg[(size_t)(nrow[s] + m) * KG + kg]);
        }
        f32x4 nc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int d = 0; d < 4; ++d) nc = mfma16(__builtin_bit_cast(bf16x8, av[d]), bneg, nc);
#pragma unroll
        for (int s = 0; s < kNSub; ++s) {
            f32x4 t = nc;
#pragma unroll
            for (int d = 0; d < 4; ++d)
                t = mfma16(__builtin_bit_cast(bf16x8, av[d]), unpack_codes(wv[s][d]), t);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[s][i] = __builtin_fmaf(sc[s], t[i], acc[s][i]);
        }
    }

#pragma unroll
    for (int s = 0; s < kNSub; ++s) red[wave][s][l] = acc[s];
    __syncthreads();

    if (ACT == MOE_ACT_SWIGLU) {
        constexpr int half = kNSub / 2;
        if (wave >= half) return;
        f32x4 gt = red[0][wave][l], up = red[0][wave + half][l];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            gt += red[w][wave][l];
            up += red[w][wave + half][l];
        }
        const int Nh = N >> 1;
        const int n = nrow[wave] + m;  // gate row == output column
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int mm = 4 * q + i;
            if (mm < mrows) {
                const float gv = gt[i];
                const float h = gv * up[i] / (1.0f + __expf(-gv));
                out[(size_t)(m0 + mm) * Nh + n] = f32_to_bf16(h);
            }
        }
    } else {
        f32x4 v = red[0][wave][l];
#pragma unroll
        for (int w = 1; w < 4; ++w) v += red[w][wave][l];
        const int n = nrow[wave] + m;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int mm = 4 * q + i;
            if (mm < mrows) out[(size_t)(m0 + mm) * N + n] = f32_to_bf16(v[i]);
        }
    }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_w4a16_grouped_gemm(const moe_layer_desc *desc, int32_t T,
                                             const uint16_t *a, const int32_t *a_gather,
                                             int32_t n_src, int32_t N, int32_t K,
                                             const uint8_t *w_packed, const uint16_t *w_scales,
                                             const int32_t *group_offsets, int32_t act,
                                             uint16_t *out, void *stream) {
    MOE_TRY(check_desc(desc));
    MOE_TRY(check_tokens(T));
    if (act != MOE_ACT_NONE && act != MOE_ACT_SWIGLU) return MOE_ERR_UNSUPPORTED;
    if (N < 64 || N % 64 || K < 128 || K % 128 || N > 65536 || K > 65536) return MOE_ERR_SHAPE;
    if (act == MOE_ACT_SWIGLU && (N / 2) % 32) return MOE_ERR_SHAPE;
    if (a_gather && (n_src < 0 || n_src > MOE_MAX_TOKENS)) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    if (!a || !w_packed || !w_scales || !group_offsets || !out) return MOE_ERR_NULL;
    if (!aligned(a, 16) || !aligned(w_packed, 16) || !aligned(w_scales, 2) ||
        !aligned(group_offsets, 4) || !aligned(out, 16) || (a_gather && !aligned(a_gather, 4)))
        return MOE_ERR_ALIGN;
    const int G = desc->n_routed + desc->n_shared;
    const int64_t R = (int64_t)T * (desc->top_k + desc->n_shared);
    const int64_t max_tiles = R / kRowsPerTile + (R < G ? R : G);
    const int NB = N / (16 * kNSub);
    const int64_t blocks = max_tiles * NB;
    if (blocks > 0x7FFFFFFF) return MOE_ERR_SHAPE;
    hipStream_t st = (hipStream_t)stream;
    if (act == MOE_ACT_SWIGLU)
        hipLaunchKernelGGL(k_w4a16_stream<MOE_ACT_SWIGLU>, dim3((unsigned)blocks), dim3(256), 0, st,
                           a, a_gather, n_src, (const u32x4 *)w_packed, w_scales, group_offsets, G,
                           (int)R, N, K, out, NB);
    else
        hipLaunchKernelGGL(k_w4a16_stream<MOE_ACT_NONE>, dim3((unsigned)blocks), dim3(256), 0, st, a,
                           a_gather, n_src, (const u32x4 *)w_packed, w_scales, group_offsets, G,
                           (int)R, N, K, out, NB);
    return launch_status();
}
