// moe_mx_gemm.hip -- fp8 activations on gfx950's block-scaled matrix cores.
//
// Two variants the pages name next to the W4A16 path:
//   * W4A8 experts: the 4-bit expert weights upcast to fp8 and multiplied
//     with e4m3 activations scaled per token per 128 elements, the per-128
//     input scales applied on the accumulator ("Throughputmaxxing:
//     DeepSeek-V4-Flash on Isambard-AI", "A pass through the model");
//   * FP8_BLOCK projections: e4m3 weights with one scale per 128x128 block
//     and dynamic activation scales in ue8m0 format (model card
//     "canada-quant/DeepSeek-V4-Flash-W4A16-FP8-MTP", "Component precisions").
// On gfx950 both are one instruction: v_mfma_scale_f32_16x16x128_f8f6f4
// multiplies a 16x128 fp8 tile by a 128x16 fp8 or FP4 (E2M1) tile and applies
// one UE8M0 scale per row (or column) per 32 k on each side, exactly, before
// the fp32 accumulation.  The FP4 expert weights (E2M1, UE8M0 per 32) are its
// operand as they are stored -- the "upcast to fp8" costs no instruction --
// and the activation scales (powers of two, per 128) ride on the same
// instruction, so the k loop has no unpacking and no scale arithmetic.
//
// moe_act_quant_fp8: bf16 rows -> e4m3 codes + UE8M0 scale per 128.
// k_mx_gemm: a 128 x 256 tile (permuted rows x weight rows) of one group
// per workgroup of eight waves, each wave all 128 rows (eight 16-row
// m-tiles) by 32 weight rows (two 16-row subtiles).  Per 128-wide k group
// the activation tile (128 rows x 128 bytes) goes from global memory
// straight into one of three LDS stages (global_load_lds), two k groups
// ahead; each wave loads its weight subtiles into registers two k groups
// ahead.  m-tiles past the group's rows are skipped.
#include <type_traits>

#include "moe_gemm_common.h"

namespace moe {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kMxTM = 128;     // permuted rows per tile
constexpr int kMxTN = 256;     // weight rows per tile
constexpr int kMxWaves = 8;
constexpr int kMxStages = 3;   // activation stages in LDS
constexpr int kMxMaxKG = 32;   // K <= 4096 (the activation scales of a tile sit in LDS)
constexpr int kBFp8 = 0, kBFp4 = 4;  // operand formats of the instruction (e4m3, E2M1)

// Where the 16-byte chunk c of row r of an activation stage sits: chunk
// c ^ mx_swz(r).  A lane of an operand read takes chunks q and q + 4 of row
// r (q = lane / 16); gfx950 serves a 16-byte-per-lane read 16 lanes per
// cycle, the lanes grouped as {0-3, 12-15, 20-23, 24-27}, {4-11, 16-19,
// 28-31} and the same plus 32.  Two 128-byte rows share the 256 bytes of
// the 64 banks; (r >> 1) & 7 puts the eight rows of each parity that one
// group reads on eight distinct chunks.
__device__ __forceinline__ int mx_swz(int r) { return (r >> 1) & 7; }

// The UE8M0 code of the activation scale of a block whose max |x| is amax
// (a finite non-negative fp32): the smallest e with amax <= 448 * 2^e,
// clamped to [-127, 127], plus 127; 127 for amax = 0.  amax = m 2^E with m
// in [1, 2): e = E - 8 when m <= 1.75 (448 = 1.75 2^8), else E - 7.
__device__ __forceinline__ int act_scale_code(float amax) {
    const uint32_t b = __float_as_uint(amax);
    if (b == 0u) return 127;
    const int ex = (int)(b >> 23);
    if (ex == 0) return 0;  // below 2^-126: the smallest scale
    int e = ex - 127 - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    e = max(e, -127);
    return e + 127;
}

// rows x K bf16 -> e4m3 codes and one UE8M0 scale per 128 consecutive
// elements of a row.  Sixteen lanes take one 128-element block (eight
// elements each), so a wave takes four blocks.
__global__ __launch_bounds__(256) void k_act_quant(const uint16_t *__restrict__ a, int rows, int K,
                                                   uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
    const int l = lane_id(), wave = threadIdx.x >> 6;
    const int KB = K >> 7;
    const long long blk = (long long)blockIdx.x * 16 + wave * 4 + (l >> 4);
    const bool in = blk < (long long)rows * KB;
    const long long row = in ? blk / KB : 0;
    const int kb = in ? (int)(blk - row * KB) : 0;
    const size_t off = (size_t)row * K + 128 * kb + 8 * (l & 15);
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (in) v = *(const u32x4 *)(a + off);
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(v[i] << 16);
        x[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, kWave));
    const int E = act_scale_code(amax);
    const float inv = __uint_as_float((uint32_t)(254 - E) << 23);  // 2^-(E-127): exact
    uint32_t w0 = 0u, w1 = 0u;
    w0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[0] * inv, x[1] * inv, (int)w0, false);
    w0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[2] * inv, x[3] * inv, (int)w0, true);
    w1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[4] * inv, x[5] * inv, (int)w1, false);
    w1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[6] * inv, x[7] * inv, (int)w1, true);
    if (in) {
        *(uint2 *)(codes + off) = make_uint2(w0, w1);
        if ((l & 15) == 0) scales[(size_t)row * KB + kb] = (uint8_t)E;
    }
}

struct MxArgs {
    const uint8_t *a;         // e4m3 codes [n_src or R][K]
    const uint8_t *as;        // UE8M0 [n_src or R][K/128]
    const int32_t *gather;    // row r reads a[gather[r]] (or null: a[r])
    int n_src;
    const uint8_t *wq;        // weights in the kernel layout
    const uint8_t *ws;        // FP4: UE8M0 [G][N][K/32]; FP8: UE8M0 [N/128][K/128]
    const int32_t *offsets;   // group offsets [G+1]; null: one group of rows [0, R)
    int G, R, N, K;
    uint16_t *out;            // bf16 [R][N] or [R][N/2] (SwiGLU)
    int NB;                   // n-blocks of 256 weight rows
};

template <int BF, int ACT>
__global__ __launch_bounds__(512) void k_mx_gemm(MxArgs p) {
    constexpr int MT = kMxTM / 16;                        // m-tiles per wave
    constexpr int WDW = BF == kBFp4 ? 4 : 8;              // weight dwords per lane per subtile
    constexpr int NLB = BF == kBFp4 ? 4 : 4;              // vector loads of one load_b (FP8 scales are scalar)
    constexpr int NLA = kMxTM * 128 / 1024 / kMxWaves;    // activation loads per wave per k group (2)
    __shared__ u32x4 sA[kMxStages][kMxTM * 8];
    __shared__ uint8_t sAs[kMxMaxKG * kMxTM];             // [kg][row]
    __shared__ int srow[kMxTM];
    const int tid = threadIdx.x, wave = tid >> 6, l = lane_id();
    const int m = l & 15, q = l >> 4;
    int g, m0, mrows, nb;
    if (!find_tile_item(blockIdx.x, p.NB, kMxTM, p.offsets, p.G, g, m0, mrows, nb, p.R)) return;  // uniform
    if (m0 < 0 || m0 >= p.R) return;
    g = __builtin_amdgcn_readfirstlane(g);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    nb = __builtin_amdgcn_readfirstlane(nb);
    mrows = __builtin_amdgcn_readfirstlane(min(mrows, p.R - m0));
    const int K = p.K, N = p.N, KG = K >> 7, NT = N >> 4;

    // the wave's two weight subtiles: SwiGLU gate and up rows of the same 16
    // output columns; otherwise 32 consecutive rows
    int wrow[2];
    if (ACT == MOE_ACT_SWIGLU) {
        wrow[0] = nb * (kMxTN / 2) + 16 * wave;
        wrow[1] = (N >> 1) + wrow[0];
    } else {
        wrow[0] = nb * kMxTN + 32 * wave;
        wrow[1] = wrow[0] + 16;
    }

    if (tid < kMxTM) {
        int sr = -1;
        if (tid < mrows) {
            if (p.gather) {
                const int t = p.gather[m0 + tid];
                sr = (unsigned)t < (unsigned)p.n_src ? t : -1;
            } else {
                sr = m0 + tid;
            }
        }
        srow[tid] = sr;
    }
    __syncthreads();
    for (int i = tid; i < kMxTM * KG; i += 512) {  // the tile's activation scales, [kg][row]
        const int r = i & (kMxTM - 1), kg = i >> 7;
        sAs[i] = p.as[(size_t)max(srow[r], 0) * KG + kg];
    }
    __syncthreads();

    // activation loads: wave w moves rows 16w .. 16w+15, two loads of eight
    // rows (rows without a source read row 0 and are never stored)
    uint32_t aoff[NLA];
#pragma unroll
    for (int j = 0; j < NLA; ++j) {
        const int r = 16 * wave + 8 * j + (l >> 3);
        const int c = (l & 7) ^ mx_swz(r);
        aoff[j] = (uint32_t)max(srow[r], 0) * (uint32_t)K + 16 * c;
    }
    auto dma_a = [&](auto stage, int kg) {
        u32x4 *A = sA[decltype(stage)::value];
#pragma unroll
        for (int j = 0; j < NLA; ++j)
            dma16_untracked(p.a + (size_t)aoff[j] + (size_t)kg * 128, &A[(16 * wave + 8 * j) * 8]);
    };
    // weights: subtile s of k group kg; FP4 blocks of 1 KB (lane l: 16
    // bytes), FP8 blocks of 2 KB (lane l: 32 bytes)
    const u32x4 *wsrc[2];
    const uint8_t *ssrc[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const size_t blk0 = ((size_t)g * NT + (wrow[s] >> 4)) * KG;
        wsrc[s] = (const u32x4 *)p.wq + blk0 * (WDW / 4) * kWave + (WDW / 4) * l;
        ssrc[s] = BF == kBFp4 ? p.ws + ((size_t)g * N + wrow[s] + m) * (K >> 5) + q
                              : p.ws + (size_t)(wrow[s] >> 7) * KG;
    }
    auto load_b = [&](int kg, v8i (&b)[2], int (&bs)[2]) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const u32x4 *src = wsrc[s] + (size_t)kg * (WDW / 4) * kWave;
            const u32x4 lo = src[0];
            b[s][0] = (int)lo[0]; b[s][1] = (int)lo[1]; b[s][2] = (int)lo[2]; b[s][3] = (int)lo[3];
            if constexpr (BF == kBFp8) {
                const u32x4 hi = src[1];
                b[s][4] = (int)hi[0]; b[s][5] = (int)hi[1]; b[s][6] = (int)hi[2]; b[s][7] = (int)hi[3];
            } else {
                b[s][4] = b[s][5] = b[s][6] = b[s][7] = 0;
            }
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) bs[s] = BF == kBFp4 ? (int)ssrc[s][kg * 4] : (int)ssrc[s][kg];
    };

    f32x4 acc[MT][2];
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    v8i bw[3][2];
    int bsc[3][2];

    // in flight before the loop: activations of k groups 0 and 1 (stages 0
    // and 1), weights of k groups 0 and 1 (buffers 0 and 1)
    const int k1 = min(1, KG - 1);
    dma_a(std::integral_constant<int, 0>(), 0);
    load_b(0, bw[0], bsc[0]);
    dma_a(std::integral_constant<int, 1>(), k1);
    load_b(k1, bw[1], bsc[1]);

    // step kg: activations in stage kg % 3, weights in buffer kg % 3; it
    // first issues k group kg+2 into stage and buffer (kg+2) % 3 (the ones
    // step kg-1 used: every wave is past it after the barrier).  Past the
    // end the loads repeat the last k group (never read).
    auto step = [&](auto st, int kg) {
        constexpr int S = decltype(st)::value, SN = (S + 2) % 3;
        // the loads of k group kg (activations and weights) have landed;
        // those of kg+1 may still be in flight
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(NLA + NLB));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        const int k2 = min(kg + 2, KG - 1);
        dma_a(std::integral_constant<int, SN>(), k2);
        load_b(k2, bw[SN], bsc[SN]);
        const u32x4 *A = sA[S];
        const uint8_t *As = sAs + kg * kMxTM;
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) {
            if (16 * mi >= mrows) break;  // uniform: the m-tiles past the group's rows
            const int r = 16 * mi + m;
            const u32x4 a0 = A[r * 8 + (q ^ mx_swz(r))];
            const u32x4 a1 = A[r * 8 + ((q + 4) ^ mx_swz(r))];
            const v8i av = v8i{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                               (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
            const int sa = As[r];
#pragma unroll
            for (int s = 0; s < 2; ++s)
                acc[mi][s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bw[S][s], acc[mi][s], kBFp8,
                                                                              BF, 0, sa, 0, bsc[S][s]);
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    for (int kg = 0; kg < KG; kg += 3) {
        step(I0(), kg);
        if (kg + 1 >= KG) break;
        step(I1(), kg + 1);
        if (kg + 2 >= KG) break;
        step(I2(), kg + 2);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load into LDS outlives the block

    // epilogue: lane (m, q) holds column m of each subtile, rows 4q..4q+3 of
    // each m-tile
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * mi + 4 * q + i;
            if (row >= mrows) continue;
            const bool live = srow[row] >= 0;  // a row without a source is zero
            if (ACT == MOE_ACT_SWIGLU) {
                const float gv = acc[mi][0][i], uv = acc[mi][1][i];
                const float hv = gv * uv * __frcp_rn(1.0f + __expf(-gv));
                p.out[(size_t)(m0 + row) * (N >> 1) + wrow[0] + m] = live ? f32_to_bf16(hv) : (uint16_t)0;
            } else {
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    p.out[(size_t)(m0 + row) * N + wrow[s] + m] = live ? f32_to_bf16(acc[mi][s][i]) : (uint16_t)0;
            }
        }
    }
}

// canonical e4m3 weights [N][K] -> 2 KB blocks per (16 rows, 128-wide k
// group): block (nt, kg) at (nt*K/128 + kg)*2048, lane l = (n % 16) + 16q
// owns bytes [32l, 32l+32): k = 128kg + 16q + [0, 16), then 128kg + 64 +
// 16q + [0, 16) (the order in which the instruction reads an fp8 operand)
__global__ void k_fp8_prepack(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int N, int K) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;  // one 16-byte piece each
    const long long total = (long long)N * K / 16;
    if (i >= total) return;
    const int KG = K >> 7;
    const long long blk = i >> 7;     // 128 pieces per 2 KB block
    const int piece = (int)(i & 127);
    const int lane = piece >> 1, half = piece & 1;
    const int nt = (int)(blk / KG), kg = (int)(blk - (long long)nt * KG);
    const int n = 16 * nt + (lane & 15), qq = lane >> 4;
    const int k = 128 * kg + 64 * half + 16 * qq;
    *(u32x4 *)(dst + 16 * i) = *(const u32x4 *)(src + (size_t)n * K + k);
}

template <int BF>
void launch_mx(int act, const MxArgs &a, hipStream_t st) {
    const int64_t max_tiles = (int64_t)a.R / kMxTM + (a.R < a.G ? a.R : a.G);
    const int64_t blocks = (max_tiles * a.NB + 7) / 8 * 8;  // a whole slice per XCD
    if (act == MOE_ACT_SWIGLU)
        hipLaunchKernelGGL((k_mx_gemm<BF, MOE_ACT_SWIGLU>), dim3((unsigned)blocks), dim3(512), 0, st, a);
    else
        hipLaunchKernelGGL((k_mx_gemm<BF, MOE_ACT_NONE>), dim3((unsigned)blocks), dim3(512), 0, st, a);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_act_quant_fp8(int32_t rows, int32_t K, const uint16_t *a, uint8_t *codes,
                                        uint8_t *scales, void *stream) {
    if (rows < 0 || rows > MOE_MAX_TOKENS * 9 || K < 128 || K % 128 || K > 65536) return MOE_ERR_SHAPE;
    if (rows == 0) return MOE_OK;
    if (!a || !codes || !scales) return MOE_ERR_NULL;
    if (!aligned(a, 16) || !aligned(codes, 8)) return MOE_ERR_ALIGN;
    const long long blocks = (long long)rows * (K / 128);
    hipLaunchKernelGGL(k_act_quant, dim3((unsigned)((blocks + 15) / 16)), dim3(256), 0, (hipStream_t)stream, a,
                       rows, K, codes, scales);
    return launch_status();
}

extern "C" moe_status moe_w4a8_grouped_gemm(const moe_layer_desc *desc, int32_t T, const uint8_t *a,
                                            const uint8_t *a_scales, const int32_t *a_gather, int32_t n_src,
                                            int32_t N, int32_t K, const uint8_t *w_packed,
                                            const uint8_t *w_scales, const int32_t *group_offsets,
                                            int32_t act, uint16_t *out, void *stream) {
    MOE_TRY(check_desc(desc));
    MOE_TRY(check_tokens(T));
    if (act != MOE_ACT_NONE && act != MOE_ACT_SWIGLU) return MOE_ERR_UNSUPPORTED;
    if (N < kMxTN || N % kMxTN || K < 128 || K % 128 || N > 65536 || K > 128 * kMxMaxKG) return MOE_ERR_SHAPE;
    if (a_gather && (n_src < 1 || n_src > MOE_MAX_TOKENS)) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    if (!a || !a_scales || !w_packed || !w_scales || !group_offsets || !out) return MOE_ERR_NULL;
    if (!aligned(a, 16) || !aligned(w_packed, 16) || !aligned(out, 4) || !aligned(group_offsets, 4) ||
        (a_gather && !aligned(a_gather, 4)))
        return MOE_ERR_ALIGN;
    MxArgs x{a, a_scales, a_gather, n_src, w_packed, w_scales, group_offsets,
             desc->n_routed + desc->n_shared, T * (desc->top_k + desc->n_shared), N, K, out, N / kMxTN};
    const int64_t max_tiles = (int64_t)x.R / kMxTM + (x.R < x.G ? x.R : x.G);
    if (max_tiles * x.NB > 0x7FFFFFF0) return MOE_ERR_SHAPE;
    launch_mx<kBFp4>(act, x, (hipStream_t)stream);
    return launch_status();
}

extern "C" moe_status moe_fp8_block_gemm(int32_t M, int32_t N, int32_t K, const uint8_t *a,
                                         const uint8_t *a_scales, const uint8_t *w_packed,
                                         const uint8_t *w_scales, uint16_t *out, void *stream) {
    if (M < 0 || M > MOE_MAX_TOKENS || N < kMxTN || N % kMxTN || N > 65536 || K < 128 || K % 128 ||
        K > 128 * kMxMaxKG)
        return MOE_ERR_SHAPE;
    if (M == 0) return MOE_OK;
    if (!a || !a_scales || !w_packed || !w_scales || !out) return MOE_ERR_NULL;
    if (!aligned(a, 16) || !aligned(w_packed, 16) || !aligned(out, 4)) return MOE_ERR_ALIGN;
    MxArgs x{a, a_scales, nullptr, M, w_packed, w_scales, nullptr, 1, M, N, K, out, N / kMxTN};
    launch_mx<kBFp8>(MOE_ACT_NONE, x, (hipStream_t)stream);
    return launch_status();
}

extern "C" moe_status moe_fp8_prepack(int32_t N, int32_t K, const uint8_t *w_canonical, uint8_t *w_packed,
                                      void *stream) {
    if (N < 16 || N % 16 || K < 128 || K % 128 || (int64_t)N * K > ((int64_t)1 << 34)) return MOE_ERR_SHAPE;
    if (!w_canonical || !w_packed) return MOE_ERR_NULL;
    if (!aligned(w_canonical, 16) || !aligned(w_packed, 16)) return MOE_ERR_ALIGN;
    const size_t bytes = (size_t)N * K;
    const uintptr_t s0 = (uintptr_t)w_canonical, d0 = (uintptr_t)w_packed;
    if (s0 < d0 + bytes && d0 < s0 + bytes) return MOE_ERR_SHAPE;  // overlapping buffers
    const long long pieces = (long long)bytes / 16;
    hipLaunchKernelGGL(k_fp8_prepack, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                       w_canonical, w_packed, N, K);
    return launch_status();
}
