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
// per workgroup of eight waves, 2 x 4 (rows x weight rows): each wave takes
// a 64-row half (four 16-row m-tiles) and four 16-row weight subtiles.  Per
// 128-wide k group the activation tile (128 rows x 128 bytes), the 16 weight
// subtiles and the FP4 scale bytes go from global memory straight into one
// of three LDS stages (global_load_lds), two k groups ahead.  A work item
// multiplies a fixed number of m-tiles per wave (4, 2 or none), chosen from
// its row count.
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

// A per-lane LDS offset the compiler cannot precompute: passed through an
// empty asm once per k step, each read's address is then the stage array plus
// this register plus a constant that fits the instruction's immediate (LDS
// past 64 KB does not fit one, so otherwise every read's full address is
// computed ahead and held in a register of its own for the whole k loop).
// The offset, not the pointer, is laundered: the reads stay reads of the
// stage's own array, so the compiler still tells the stages apart and does
// not wait for the loads into the others.
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

constexpr int kMxTM = 128;     // permuted rows per tile
constexpr int kMxTN = 256;     // weight rows per tile (FP8 weights; FP4 weights take 512 when N allows)
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

// rows x K bf16 -> e4m3 codes and one UE8M0 scale per 128 consecutive
// elements of a row.  Sixteen lanes take one 128-element block (eight
// elements each), so a wave takes four blocks.  DEQ: also each code times
// its scale as bf16 (exact: four significant bits times a power of two)
template <bool DEQ>
__global__ __launch_bounds__(256) void k_act_quant(const uint16_t *__restrict__ a, int rows, int K,
                                                   uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                                   uint16_t *__restrict__ deq) {
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
    if constexpr (DEQ) {
        const float s = ue8m0_to_f32((uint32_t)E);
        const int c0 = (int)w0, c1 = (int)w1;
        const u32x4 d = u32x4{pack_bf16x2(__builtin_amdgcn_cvt_f32_fp8(c0, 0) * s, __builtin_amdgcn_cvt_f32_fp8(c0, 1) * s),
                              pack_bf16x2(__builtin_amdgcn_cvt_f32_fp8(c0, 2) * s, __builtin_amdgcn_cvt_f32_fp8(c0, 3) * s),
                              pack_bf16x2(__builtin_amdgcn_cvt_f32_fp8(c1, 0) * s, __builtin_amdgcn_cvt_f32_fp8(c1, 1) * s),
                              pack_bf16x2(__builtin_amdgcn_cvt_f32_fp8(c1, 2) * s, __builtin_amdgcn_cvt_f32_fp8(c1, 3) * s)};
        if (in) *(u32x4 *)(deq + off) = d;
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
    int NB;                   // n-blocks of TN weight rows (the instance's tile width)
};

// KGC: the k groups of K when the instance is unrolled for them (16 or 32,
// the layer's K of 2048 and 4096: the compiler then counts the loads in
// flight exactly), 0 for any K (a runtime loop, compiled apart so that its
// register allocation does not reach the unrolled instances).
// NSW: 16-row weight subtiles per wave, 4 or 8; the tile is 64 NSW weight
// rows wide.  With 8 (FP4 weights) a wave multiplies 64 rows by 128 weight
// rows: its 128 accumulators live in AGPRs (nothing but the matrix cores
// touches them before the epilogue) and every activation operand it reads
// from LDS feeds twice the matrix instructions.  On gfx950 a wave's LDS
// reads into registers do not overlap its SIMD's matrix instructions (a
// 1 KB read costs 25-40 SIMD cycles, measured), so operand bytes read per
// instruction set the pace: 512 per 16x16x128 instruction here against 768
// with 4 subtiles.
template <int BF, int ACT, int KGC, int NSW>
__global__ __launch_bounds__(512) void k_mx_gemm(MxArgs p) {
    constexpr int MT = kMxTM / 32;                        // m-tiles per wave (a row half of the tile)
    constexpr int TN = 64 * NSW;                          // weight rows per tile
    constexpr int NSUB = TN / 16;                         // weight subtiles per tile
    constexpr int WB = BF == kBFp4 ? 1024 : 2048;         // bytes of one 16-row weight subtile per k group
    constexpr int WQ = WB / 1024;                         // 1 KB loads per subtile
    typedef int wvec __attribute__((ext_vector_type(4 * WQ)));
    constexpr int NLA = kMxTM * 128 / 1024 / kMxWaves;    // activation loads per wave per k group (2)
    constexpr int NBW = NSUB / kMxWaves;                  // weight subtiles each wave loads (2 or 4)
    constexpr int NLB = NBW * WQ + (BF == kBFp4 ? 1 : 0); // weight (and FP4 scale) loads per wave
    constexpr int SRW = TN / kMxWaves;                    // FP4 scale rows each wave loads (32 or 64)
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
    __shared__ u32x4 sB0[NSUB * WB / 16], sB1[NSUB * WB / 16], sB2[NSUB * WB / 16];
    // FP4 weight scales: wave w's load fills words 64w .. 64w+63 with tile
    // rows SRW w .. SRW w + SRW - 1 (with SRW = 32, lanes 32..63 load a copy:
    // an unconditional load keeps the wait counts exact)
    __shared__ uint32_t sS0[BF == kBFp4 ? 64 * kMxWaves : 1], sS1[BF == kBFp4 ? 64 * kMxWaves : 1],
        sS2[BF == kBFp4 ? 64 * kMxWaves : 1];
    // activation scales, [kg][m][mi] = row 16 mi + m: a lane's eight m-tile
    // scales of one k group are one 8-byte read (four of them its half's)
    __shared__ __attribute__((aligned(8))) uint8_t sAs[kMxMaxKG * kMxTM];
    __shared__ int srow[kMxTM];
    // With 8 subtiles per wave the accumulators go to AGPRs: the compiler
    // allocates none unless the kernel names one (it then splits the 256
    // registers of a wave between the two files)
    if constexpr (NSW == 8) asm volatile("" ::: "a0");
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), l = lane_id();
    const int m = l & 15, q = l >> 4;
    TileItem it;
    if (!workgroup_tile_item(p.NB, kMxTM, p.offsets, p.G, p.R, it)) return;  // the whole workgroup: no work item
    const int g = it.g, m0 = it.m0, mrows = it.mrows, nb = it.nb;
    const int K = p.K, N = p.N, KG = KGC ? KGC : K >> 7, NT = N >> 4;

    // the tile's NSUB weight subtiles: SwiGLU gate rows of TN/2 output
    // columns (t < NSUB/2) and the up rows of the same columns (t >=
    // NSUB/2); otherwise TN consecutive rows.  Waves are 2 x 4 (rows x weight
    // rows): wave w takes row half wm = w / 4 (four 16-row m-tiles) and, with
    // wn = w % 4, NSW subtiles: gate subtiles (NSW/2) wn .. and their up rows
    // (SwiGLU: 8 NSW output columns) or NSW wn .. NSW wn + NSW - 1.
    constexpr int GS = NSUB / 2;  // gate subtiles (SwiGLU)
    const int wm = wave >> 2, wn = wave & 3;
    auto subtile_row = [&](int t) {
        if (ACT == MOE_ACT_SWIGLU) return (t >= GS ? (N >> 1) : 0) + nb * (TN / 2) + 16 * (t % GS);
        return nb * TN + 16 * t;
    };
    // subtile j of the wave is tsb + tofs(j): a wave base and a constant, so
    // that every operand address is one register plus an immediate offset
    const int tsb = (ACT == MOE_ACT_SWIGLU ? NSW / 2 : NSW) * wn;
    auto tofs = [](int j) { return ACT == MOE_ACT_SWIGLU ? (j < NSW / 2 ? j : GS + j - NSW / 2) : j; };
    int ts[NSW];
#pragma unroll
    for (int j = 0; j < NSW; ++j) ts[j] = tsb + tofs(j);
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
    size_t aoff[NLA];  // 64-bit: rows x K of a can pass 2^32 elements
#pragma unroll
    for (int j = 0; j < NLA; ++j) {
        const int r = 16 * wave + 8 * j + (l >> 3);
        const int c = (l & 7) ^ mx_swz(r);
        aoff[j] = (size_t)max(srow[r], 0) * K + 16 * c;
    }
    // weight loads: wave w moves subtiles NBW w .. NBW w + NBW - 1 (their k
    // group's blocks are WB contiguous bytes each); FP4 scales: lane l moves
    // the four UE8M0 bytes of tile row SRW w + l % SRW
    const uint8_t *bsrc[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j)
        bsrc[j] = p.wq + ((size_t)g * NT + (subtile_row(NBW * wave + j) >> 4)) * KG * WB + 16 * l;
    const int srt = SRW * wave + (l % SRW);
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
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int h = 0; h < WQ; ++h)
                dma16(bsrc[j] + (size_t)kg * WB + 1024 * h, &B[((NBW * wave + j) * WB + 1024 * h) / 16]);
        if constexpr (BF == kBFp4)
            __builtin_amdgcn_global_load_lds(ssrc + 4 * kg, (lds_void_t *)&S[64 * wave], 4, 0, 0);
    };

    // per-lane LDS offsets of the operand reads (u32x4 units for A and B,
    // bytes for the scales)
    const int a_lane0 = (64 * wm + m) * 8 + (q ^ mx_swz(m)), a_lane1 = (64 * wm + m) * 8 + ((q + 4) ^ mx_swz(m));
    const int b_base = l + tsb * (WB / 16);
    // FP4 scale of tile row rt = 16 ts + m sits in word (rt / SRW) 64 +
    // rt % SRW, byte q; 16 tsb is a multiple of SRW, so the wave's part
    // separates from subtile j's constant part
    const int s_base = (64 * (16 * tsb / SRW) + m) * 4 + q;
    auto s_ofs = [](int j) {
        const int c = ACT == MOE_ACT_SWIGLU ? (j < NSW / 2 ? j : NSUB / 2 + j - NSW / 2) : j;
        return 4 * (64 * ((16 * c) / SRW) + (16 * c) % SRW);
    };
    const int sa_lane = m * 8 + 4 * wm;
    f32x4 acc[MT][NSW];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NSW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

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
        const uint32_t sab = *(const uint32_t *)(sAs + sa_lane + kg * kMxTM);
        // per-step operand bases (the wide instance launders them, see
        // opaque_lds; the 4-subtile one fits its registers as it is)
        const u32x4 *Bp = B + (NSW == 8 ? opaque(b_base) : b_base);
        const uint8_t *Sp = Sc + (NSW == 8 ? opaque(s_base) : s_base);
        auto read_b = [&](int j, wvec &bv, int &bs) {
#pragma unroll
            for (int h = 0; h < WQ; ++h) {
                const u32x4 w = Bp[(tofs(j) * WB + 1024 * h) / 16];
#pragma unroll
                for (int i = 0; i < 4; ++i) bv[4 * h + i] = (int)w[i];
            }
            if constexpr (BF == kBFp4)
                bs = Sp[s_ofs(j)];
            else
                bs = p.ws[(size_t)(subtile_row(ts[j]) >> 7) * KG + kg];
        };
        auto mfma = [&](const v8i &a, const wvec &b, f32x4 &c, int sa, int sb) {
            if constexpr (BF == kBFp4)
                c = mfma_scale_fp8_fp4(a, b, c, kBFp8, BF, 0, sa, 0, sb);
            else
                c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, kBFp8, BF, 0, sa, 0, sb);
        };
        v8i av[MTA > 0 ? MTA : 1];
        const u32x4 *A0p = A + (NSW == 8 ? opaque(a_lane0) : a_lane0);
        const u32x4 *A1p = A + (NSW == 8 ? opaque(a_lane1) : a_lane1);
        auto read_a = [&]() {
#pragma unroll
            for (int mi = 0; mi < MTA; ++mi) {
                const u32x4 a0 = A0p[128 * mi];
                const u32x4 a1 = A1p[128 * mi];
                av[mi] = v8i{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                             (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
            }
        };
        if constexpr (NSW == 4) {
            // every operand read at once (one wait for the LDS round trip
            // per step), then the step's matrix instructions back to back
            wvec bv[NSW];
            int bs[NSW];
#pragma unroll
            for (int j = 0; j < NSW; ++j) read_b(j, bv[j], bs[j]);
            read_a();
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * MTA + NSW * WQ + NSW + 1, 0);
#pragma unroll
            for (int mi = 0; mi < MTA; ++mi) {
                const int sa = (int)((sab >> (8 * mi)) & 0xFFu);
#pragma unroll
                for (int j = 0; j < NSW; ++j) mfma(av[mi], bv[j], acc[mi][j], sa, bs[j]);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, NSW * MTA, 0);
        } else {
            // the activation operands read once; the weight operands of
            // subtile j+1 read while subtile j's matrix instructions run, so
            // only two subtiles' operands are live
            read_a();
            wvec bv0, bv1;
            int bs0, bs1;
            read_b(0, bv0, bs0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * MTA + WQ + 2, 0);
#pragma unroll
            for (int j = 0; j < NSW; ++j) {
                wvec &bc = (j & 1) ? bv1 : bv0;
                int &sc = (j & 1) ? bs1 : bs0;
                if (j + 1 < NSW) read_b(j + 1, (j & 1) ? bv0 : bv1, (j & 1) ? bs0 : bs1);
#pragma unroll
                for (int mi = 0; mi < MTA; ++mi) mfma(av[mi], bc, acc[mi][j], (int)((sab >> (8 * mi)) & 0xFFu), sc);
                if (j + 1 < NSW) __builtin_amdgcn_sched_group_barrier(0x100, WQ + 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, MTA, 0);
            }
        }
        if constexpr (NSW == 8) {
            // keep the step's matrix instructions in the step: the accumulators
            // (in AGPRs) are pinned at its end, or the instruction selector
            // moves them past the next barrier and two steps' operands live
            // at once
#pragma unroll
            for (int mi = 0; mi < MTA; ++mi)
#pragma unroll
                for (int j = 0; j < NSW; ++j) asm volatile("" : "+a"(acc[mi][j]));
        }
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

    int wrow[NSW];
#pragma unroll
    for (int j = 0; j < NSW; ++j) wrow[j] = subtile_row(ts[j]);
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
                for (int c = 0; c < NSW / 2; ++c) {
                    const float gv = acc[mi][c][i], uv = acc[mi][c + NSW / 2][i];
                    const float hv = silu_mul(gv, uv);
                    p.out[(size_t)(m0 + row) * (N >> 1) + wrow[c] + m] = live ? f32_to_bf16(hv) : (uint16_t)0;
                }
            } else {
#pragma unroll
                for (int j = 0; j < NSW; ++j)
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

template <int BF, int KGC, int NSW>
void launch_mx_k(int act, const MxArgs &a, dim3 grid, hipStream_t st) {
    if (act == MOE_ACT_SWIGLU)
        hipLaunchKernelGGL((k_mx_gemm<BF, MOE_ACT_SWIGLU, KGC, NSW>), grid, dim3(512), 0, st, a);
    else
        hipLaunchKernelGGL((k_mx_gemm<BF, MOE_ACT_NONE, KGC, NSW>), grid, dim3(512), 0, st, a);
}

// FP4 weights take 512-wide tiles when N is a multiple of 512 (the unrolled
// K = 4096 and 2048 instances) and the work list holds at least one item per
// CU with them; FP8 weights (twice the LDS per subtile), other shapes and the
// few-token calls (a handful of groups, whose 512-wide items would leave most
// CUs idle) 256-wide ones.
template <int BF>
void launch_mx(int act, MxArgs a, hipStream_t st) {
    const int64_t max_tiles = (int64_t)a.R / kMxTM + (a.R < a.G ? a.R : a.G);
    const bool wide = BF == kBFp4 && a.N % 512 == 0 && (a.K == 4096 || a.K == 2048) &&
                      max_tiles * (a.N / 512) >= 256;
    a.NB = a.N / (wide ? 512 : 256);
    const dim3 grid((unsigned)((max_tiles * a.NB + 7) / 8 * 8));  // a whole slice per XCD
    if constexpr (BF == kBFp4) {
        if (wide) {
            if (a.K == 4096)
                launch_mx_k<BF, 32, 8>(act, a, grid, st);
            else
                launch_mx_k<BF, 16, 8>(act, a, grid, st);
            return;
        }
    }
    if (a.K == 4096)
        launch_mx_k<BF, 32, 4>(act, a, grid, st);
    else if (a.K == 2048)
        launch_mx_k<BF, 16, 4>(act, a, grid, st);
    else
        launch_mx_k<BF, 0, 4>(act, a, grid, st);
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
    hipLaunchKernelGGL(k_act_quant<false>, dim3((unsigned)((blocks + 15) / 16)), dim3(256), 0,
                       (hipStream_t)stream, a, rows, K, codes, scales, nullptr);
    return launch_status();
}

extern "C" moe_status moe_act_quant_fp8_dequant(int32_t rows, int32_t K, const uint16_t *a, uint8_t *codes,
                                                uint8_t *scales, uint16_t *deq, void *stream) {
    if (rows < 0 || rows > MOE_MAX_TOKENS * 9 || K < 128 || K % 128 || K > 65536) return MOE_ERR_SHAPE;
    if (rows == 0) return MOE_OK;
    if (!a || !codes || !scales || !deq) return MOE_ERR_NULL;
    if (!aligned(a, 16) || !aligned(codes, 8) || !aligned(deq, 16)) return MOE_ERR_ALIGN;
    const size_t n = (size_t)rows * K * 2;
    if ((const char *)deq < (const char *)a + n && (const char *)a < (const char *)deq + n) return MOE_ERR_SHAPE;
    const long long blocks = (long long)rows * (K / 128);
    hipLaunchKernelGGL(k_act_quant<true>, dim3((unsigned)((blocks + 15) / 16)), dim3(256), 0,
                       (hipStream_t)stream, a, rows, K, codes, scales, deq);
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
