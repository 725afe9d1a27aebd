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
typedef int v4i __attribute__((ext_vector_type(4)));

// The same instruction with an FP4 second operand in four registers (the
// 128 E2M1 codes of a lane's column take 16 bytes): the compiler's builtin
// declares that operand with eight, half of them unused.
__device__ f32x4 mfma_scale_fp8_fp4(v8i a, v4i b, f32x4 c, int cbsz, int blgp, int opsel_a, int scale_a,
                                    int opsel_b, int scale_b)
    __asm("llvm.amdgcn.mfma.scale.f32.16x16x128.f8f6f4.v8i32.v4i32");

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

// KGC: the k groups of K when the instance is unrolled for them (16 or 32,
// the layer's K of 2048 and 4096: the compiler then counts the loads in
// flight exactly), 0 for any K (a runtime loop, compiled apart so that its
// register allocation does not reach the unrolled instances).
template <int BF, int ACT, int KGC>
__global__ __launch_bounds__(512) void k_mx_gemm(MxArgs p) {
    constexpr int MT = kMxTM / 32;                        // m-tiles per wave (a row half of the tile)
    constexpr int WB = BF == kBFp4 ? 1024 : 2048;         // bytes of one 16-row weight subtile per k group
    constexpr int WQ = WB / 1024;                         // 1 KB loads per subtile
    typedef int wvec __attribute__((ext_vector_type(4 * WQ)));
    constexpr int NLA = kMxTM * 128 / 1024 / kMxWaves;    // activation loads per wave per k group (2)
    constexpr int NLB = 2 * WQ + (BF == kBFp4 ? 1 : 0);   // weight (and FP4 scale) loads per wave
    constexpr int NL = NLA + NLB;
    // Everything a k group needs goes from global memory straight into LDS
    // (global_load_lds), two k groups ahead: the activation tile (128 rows x
    // 128 bytes), the 16 weight subtiles of the tile (as stored: 1 KB FP4 or
    // 2 KB FP8 blocks) and, for FP4, the 256 rows' four UE8M0 bytes of the k
    // group.  Registers hold only the accumulators and the current
    // operands.  One LDS variable per stage: the compiler then tells the
    // stages apart and does not wait for the loads into the others before
    // reading one.
    static_assert(kMxStages == 3, "three stage variables");
    __shared__ u32x4 sA0[kMxTM * 8], sA1[kMxTM * 8], sA2[kMxTM * 8];
    __shared__ u32x4 sB0[16 * WB / 16], sB1[16 * WB / 16], sB2[16 * WB / 16];
    // FP4 weight scales: wave w's load fills words 64w .. 64w+63, lanes 0..31
    // with tile rows 32w .. 32w+31 and lanes 32..63 with a copy (an
    // unconditional load keeps the wait counts exact)
    __shared__ uint32_t sS0[BF == kBFp4 ? 2 * kMxTN : 1], sS1[BF == kBFp4 ? 2 * kMxTN : 1],
        sS2[BF == kBFp4 ? 2 * kMxTN : 1];
    // activation scales, [kg][m][mi] = row 16 mi + m: a lane's eight m-tile
    // scales of one k group are one 8-byte read (four of them its half's)
    __shared__ __attribute__((aligned(8))) uint8_t sAs[kMxMaxKG * kMxTM];
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
    const int K = p.K, N = p.N, KG = KGC ? KGC : K >> 7, NT = N >> 4;

    // the tile's 16 weight subtiles: SwiGLU gate rows of 128 output columns
    // (t < 8) and the up rows of the same columns (t >= 8); otherwise 256
    // consecutive rows.  Waves are 2 x 4 (rows x weight rows): wave w takes
    // row half wm = w / 4 (four 16-row m-tiles) and, with wn = w % 4,
    // subtiles 2wn, 2wn+1 and their up rows 2wn+8, 2wn+9 (SwiGLU: 32 output
    // columns) or 4wn .. 4wn+3.
    const int wm = wave >> 2, wn = wave & 3;
    auto subtile_row = [&](int t) {
        if (ACT == MOE_ACT_SWIGLU) return (t >= 8 ? (N >> 1) : 0) + nb * (kMxTN / 2) + 16 * (t & 7);
        return nb * kMxTN + 16 * t;
    };
    int ts[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ts[j] = ACT == MOE_ACT_SWIGLU ? 2 * wn + (j & 1) + 8 * (j >> 1) : 4 * wn + j;
    const int mw = mrows - 64 * wm;  // rows of this wave's half that exist

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
    for (int i = tid; i < kMxTM * KG; i += 512) {  // the tile's activation scales
        const int r = i & (kMxTM - 1), kg = i >> 7;
        sAs[kg * kMxTM + (r & 15) * 8 + (r >> 4)] = p.as[(size_t)max(srow[r], 0) * KG + kg];
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
    // weight loads: wave w moves subtiles 2w and 2w + 1 (their k group's
    // blocks are WB contiguous bytes each); FP4 scales: lanes 0..31 move the
    // four UE8M0 bytes of tile rows 32w .. 32w+31
    const uint8_t *bsrc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
        bsrc[j] = p.wq + ((size_t)g * NT + (subtile_row(2 * wave + j) >> 4)) * KG * WB + 16 * l;
    const int srt = 32 * wave + (l & 31);
    const uint8_t *ssrc = p.ws + ((size_t)g * N + subtile_row(srt >> 4) + (srt & 15)) * (K >> 5);
    auto dma = [&](auto stage, int kg) {
        constexpr int ST = decltype(stage)::value;
        u32x4 *A = ST == 0 ? sA0 : ST == 1 ? sA1 : sA2;
        u32x4 *B = ST == 0 ? sB0 : ST == 1 ? sB1 : sB2;
        uint32_t *S = ST == 0 ? sS0 : ST == 1 ? sS1 : sS2;
#pragma unroll
        for (int j = 0; j < NLA; ++j)
            dma16(p.a + (size_t)aoff[j] + (size_t)kg * 128, &A[(16 * wave + 8 * j) * 8]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int h = 0; h < WQ; ++h)
                dma16(bsrc[j] + (size_t)kg * WB + 1024 * h, &B[((2 * wave + j) * WB + 1024 * h) / 16]);
        if constexpr (BF == kBFp4)
            __builtin_amdgcn_global_load_lds(ssrc + 4 * kg, (lds_void_t *)&S[64 * wave], 4, 0, 0);
    };

    // per-lane LDS offsets of the operand reads (u32x4 units for A and B,
    // bytes for the scales)
    const int a_lane0 = (64 * wm + m) * 8 + (q ^ mx_swz(m)), a_lane1 = (64 * wm + m) * 8 + ((q + 4) ^ mx_swz(m));
    const int b_lane = l;
    int s_lane[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int rt = 16 * ts[j] + m;  // tile row of the FP4 scale
        s_lane[j] = ((rt >> 5) * 64 + (rt & 31)) * 4 + q;
    }
    const int sa_lane = m * 8 + 4 * wm;
    f32x4 acc[MT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // in flight before the loop: k groups 0 and 1 (stages 0 and 1)
    dma(std::integral_constant<int, 0>(), 0);
    dma(std::integral_constant<int, 1>(), min(1, KG - 1));

    // step kg: stage kg % 3; it first issues k group kg+2 into stage
    // (kg+2) % 3 (the one step kg-1 read: every wave is past it after the
    // barrier).  Past the end the loads repeat the last k group (never
    // read).  MTA of the wave's four m-tiles take part: all four, the first
    // two when its rows end there, none when its half has no rows (a fixed
    // count per work item, chosen once).
    auto step = [&](auto st, auto mta, int kg) {
        constexpr int S = decltype(st)::value, SN = (S + 2) % 3, MTA = decltype(mta)::value;
        // this wave's loads of k group kg have landed (those of kg+1 may be
        // in flight); after the barrier every wave's have
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(NL));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        dma(std::integral_constant<int, SN>(), min(kg + 2, KG - 1));
        if (MTA == 0) return;  // no rows in this wave's half: loads only
        const u32x4 *A = S == 0 ? sA0 : S == 1 ? sA1 : sA2;
        const u32x4 *B = S == 0 ? sB0 : S == 1 ? sB1 : sB2;
        const uint8_t *Sc = (const uint8_t *)(S == 0 ? sS0 : S == 1 ? sS1 : sS2);
        // addresses: one lane base per operand, the rest immediate offsets
        // (a row's swizzle depends on its row within the m-tile only)
        wvec bv[4];
        int bs[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int h = 0; h < WQ; ++h) {
                const u32x4 w = B[b_lane + (ts[j] * WB + 1024 * h) / 16];
#pragma unroll
                for (int i = 0; i < 4; ++i) bv[j][4 * h + i] = (int)w[i];
            }
            if constexpr (BF == kBFp4)
                bs[j] = Sc[s_lane[j]];
            else
                bs[j] = p.ws[(size_t)(subtile_row(ts[j]) >> 7) * KG + kg];
        }
        const uint32_t sab = *(const uint32_t *)(sAs + sa_lane + kg * kMxTM);
        // every m-tile's operand read at once (one wait for the LDS round
        // trip per step), then the step's matrix instructions back to back
        v8i av[MTA > 0 ? MTA : 1];
#pragma unroll
        for (int mi = 0; mi < MTA; ++mi) {
            const u32x4 a0 = A[a_lane0 + 128 * mi];
            const u32x4 a1 = A[a_lane1 + 128 * mi];
            av[mi] = v8i{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                         (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        }
        // the step's LDS reads first, then its matrix instructions
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * MTA + 4 * WQ + 5, 0);
#pragma unroll
        for (int mi = 0; mi < MTA; ++mi) {
            const int sa = (int)((sab >> (8 * mi)) & 0xFFu);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (BF == kBFp4)
                    acc[mi][j] = mfma_scale_fp8_fp4(av[mi], bv[j], acc[mi][j], kBFp8, BF, 0, sa, 0, bs[j]);
                else
                    acc[mi][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av[mi], bv[j], acc[mi][j],
                                                                                  kBFp8, BF, 0, sa, 0, bs[j]);
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * MTA, 0);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    // the k loop: unrolled whole in the KGC instances (around a loop back
    // edge the compiler waits for every load in flight once per iteration)
    auto kloop = [&](auto mta) {
        if constexpr (KGC != 0) {
#pragma unroll
            for (int kg = 0; kg < KGC; kg += 3) {
                step(I0(), mta, kg);
                if (kg + 1 >= KGC) break;
                step(I1(), mta, kg + 1);
                if (kg + 2 >= KGC) break;
                step(I2(), mta, kg + 2);
            }
            return;
        }
        for (int kg = 0; kg < KG; kg += 3) {
            step(I0(), mta, kg);
            if (kg + 1 >= KG) break;
            step(I1(), mta, kg + 1);
            if (kg + 2 >= KG) break;
            step(I2(), mta, kg + 2);
        }
    };
    if (mw > 32)
        kloop(std::integral_constant<int, 4>());
    else if (mw > 0)
        kloop(std::integral_constant<int, 2>());
    else
        kloop(std::integral_constant<int, 0>());
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load into LDS outlives the block

    int wrow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wrow[j] = subtile_row(ts[j]);
    // epilogue: lane (m, q) holds column m of each subtile, rows 4q..4q+3 of
    // each m-tile
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 64 * wm + 16 * mi + 4 * q + i;
            if (row >= mrows) continue;
            const bool live = srow[row] >= 0;  // a row without a source is zero
            if (ACT == MOE_ACT_SWIGLU) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const float gv = acc[mi][c][i], uv = acc[mi][c + 2][i];
                    const float hv = gv * uv * __frcp_rn(1.0f + __expf(-gv));
                    p.out[(size_t)(m0 + row) * (N >> 1) + wrow[c] + m] = live ? f32_to_bf16(hv) : (uint16_t)0;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    p.out[(size_t)(m0 + row) * N + wrow[j] + m] = live ? f32_to_bf16(acc[mi][j][i]) : (uint16_t)0;
            }
        }
    }
}

// canonical e4m3 weights [N][K] -> 2 KB blocks per (16 rows, 128-wide k
// group): block (nt, kg) at (nt*K/128 + kg)*2048; lane l = (n % 16) + 16q
// owns two 16-byte pieces, half h at [1024h + 16l, 1024h + 16l + 16): k =
// 128kg + 64h + 16q + [0, 16) (the order in which the instruction reads an
// fp8 operand: its first four registers hold k 16q.., the last four 64 +
// 16q..), so each half of a block is one contiguous 1 KB wave load
__global__ void k_fp8_prepack(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int N, int K) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;  // one 16-byte piece each
    const long long total = (long long)N * K / 16;
    if (i >= total) return;
    const int KG = K >> 7;
    const long long blk = i >> 7;     // 128 pieces per 2 KB block
    const int piece = (int)(i & 127);
    const int half = piece >> 6, lane = piece & 63;
    const int nt = (int)(blk / KG), kg = (int)(blk - (long long)nt * KG);
    const int n = 16 * nt + (lane & 15), qq = lane >> 4;
    const int k = 128 * kg + 64 * half + 16 * qq;
    *(u32x4 *)(dst + 16 * i) = *(const u32x4 *)(src + (size_t)n * K + k);
}

template <int BF, int KGC>
void launch_mx_k(int act, const MxArgs &a, dim3 grid, hipStream_t st) {
    if (act == MOE_ACT_SWIGLU)
        hipLaunchKernelGGL((k_mx_gemm<BF, MOE_ACT_SWIGLU, KGC>), grid, dim3(512), 0, st, a);
    else
        hipLaunchKernelGGL((k_mx_gemm<BF, MOE_ACT_NONE, KGC>), grid, dim3(512), 0, st, a);
}

template <int BF>
void launch_mx(int act, const MxArgs &a, hipStream_t st) {
    const int64_t max_tiles = (int64_t)a.R / kMxTM + (a.R < a.G ? a.R : a.G);
    const dim3 grid((unsigned)((max_tiles * a.NB + 7) / 8 * 8));  // a whole slice per XCD
    if (a.K == 4096)
        launch_mx_k<BF, 32>(act, a, grid, st);
    else if (a.K == 2048)
        launch_mx_k<BF, 16>(act, a, grid, st);
    else
        launch_mx_k<BF, 0>(act, a, grid, st);
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
