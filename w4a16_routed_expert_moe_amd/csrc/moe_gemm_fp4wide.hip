// moe_gemm_fp4wide.hip -- the grouped GEMM for FP4 expert weights (E2M1, one
// UE8M0 scale per 32 inputs) with bf16 activations, on 128 x 512 tiles, for
// groups of many rows (prefill, large batches).
//
// Method: the release's FP4 experts multiplied with 16-bit activations
// ("Throughputmaxxing: DeepSeek-V4-Flash on Isambard-AI", "A pass through the
// model": the experts ship in fp4; "DeepSeek V4 Flash serving hardware",
// "Released precision").  v_cvt_scalef32_pk_bf16_fp4 turns two codes into
// exact bf16 with the block's power-of-two scale folded in, so the products
// accumulate straight into the output: no offset term, no per-group scaling,
// and the accumulators can live in AGPRs, which nothing but the matrix cores
// touches before the epilogue.
//
// Why this shape: on gfx950 a wave's LDS reads into registers do not overlap
// its SIMD's matrix instructions (a 1 KB wave read costs 25-40 SIMD cycles,
// measured), so the bytes read from LDS per matrix instruction set the pace.
// A wave here multiplies 64 rows by 128 weight rows: per 16x16x32 MFMA it
// reads 128 bytes of activations and 64 of weights (against 544 for a wave
// owning 128 rows x 32 weight rows), and converts one weight word per four
// MFMAs (four conversions).
//
// A workgroup of eight waves (2 x 4: row halves x weight-row quarters)
// computes 128 permuted rows x 512 weight rows of one group.  Per 128-wide k
// group the activation tile (128 gathered rows x 256 bytes, XOR-swizzled),
// the 32 weight subtiles (1 KB each, prepacked) and the 512 rows' four UE8M0
// bytes go from global memory straight into one of two LDS stages (66 KB
// each), one k group ahead.  A wave goes through a k group one 32-wide
// slice at a time: the slice's activation operands of its m-tiles, then each
// subtile's word of the slice converted and multiplied into every m-tile.
#include <type_traits>

#include "moe_gemm_common.h"

namespace moe {
namespace {

constexpr int kFwTM = 128;              // permuted rows per tile
constexpr int kFwTN = 512;              // weight rows per tile
constexpr int kFwSub = kFwTN / 16;      // weight subtiles per tile
constexpr int kFwNSW = 8;               // weight subtiles per wave

// A per-lane LDS offset laundered through an empty asm once per k step: each
// read's address is then the stage array plus this register plus a constant
// immediate (without it the compiler computes every read's full address
// ahead -- the stage arrays sit past the 64 KB an immediate reaches -- and
// holds each in a register for the whole loop).  The offset, not the pointer,
// is laundered, so the reads stay reads of the stage's own array.
__device__ __forceinline__ int opaque_off(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

// KGC: the k groups of K when the instance is unrolled for them (16 or 32,
// the layer's K of 2048 and 4096), 0 for any even K/128 (a runtime loop).
template <int ACT, int KGC>
__global__ __launch_bounds__(512) void k_mxfp4_wide(GemmArgs p) {
    // the accumulators go to AGPRs: the compiler allocates none unless the
    // kernel names one
    asm volatile("" ::: "a0");
    __shared__ u32x4 sA0[kFwTM * 16], sA1[kFwTM * 16];          // activations, 32 KB per stage
    __shared__ u32x4 sB0[kFwSub * kWave], sB1[kFwSub * kWave];  // weights, 32 KB per stage
    __shared__ uint32_t sS0[kFwTN], sS1[kFwTN];                 // tile row r's four UE8M0 bytes
    __shared__ int srow[kFwTM];
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), l = lane_id();
    const int m = l & 15, q = l >> 4;
    const int N = p.N, NT = N >> 4, K = KGC ? KGC * 128 : p.K, KG = K >> 7, NB = N / kFwTN;
    TileItem it;
    if (!workgroup_tile_item(NB, kFwTM, p.offsets, p.G, p.R, it)) return;  // the whole workgroup: no work item
    const int g = it.g, m0 = it.m0, mrows = it.mrows, nb = it.nb;

    // the tile's 32 subtiles: SwiGLU gate rows of 256 output columns (t <
    // 16) and the up rows of the same columns (t >= 16); otherwise 512
    // consecutive rows.  Wave (wm, wn) takes row half wm and subtiles tsb +
    // tofs(j): gate subtiles 4wn .. 4wn+3 and their up rows (64 output
    // columns), or 8wn .. 8wn+7.
    constexpr int GS = kFwSub / 2;
    const int wm = wave >> 2, wn = wave & 3;
    auto subtile_row = [&](int t) {
        if (ACT == MOE_ACT_SWIGLU) return (t >= GS ? (N >> 1) : 0) + nb * (kFwTN / 2) + 16 * (t % GS);
        return nb * kFwTN + 16 * t;
    };
    const int tsb = (ACT == MOE_ACT_SWIGLU ? kFwNSW / 2 : kFwNSW) * wn;
    auto tofs = [](int j) { return ACT == MOE_ACT_SWIGLU ? (j < kFwNSW / 2 ? j : GS + j - kFwNSW / 2) : j; };

    if (tid < kFwTM) {
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

    // loads into LDS, per wave and k group: four activation loads of four
    // rows (rows 16w .. 16w+15; rows without a source read row 0 and are
    // never stored), four weight subtiles (4w .. 4w+3), and the four scale
    // bytes of tile rows 64w .. 64w+63 (one word per lane)
    size_t aoff[4];  // 64-bit: rows x K of a can pass 2^32 elements
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 16 * wave + 4 * j + (l >> 4);
        const int c = (l & 15) ^ lds_swz(r);
        aoff[j] = (size_t)max(srow[r], 0) * K + 8 * c;
    }
    const u32x4 *bsrc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bsrc[j] = p.wq + ((size_t)g * NT + (subtile_row(4 * wave + j) >> 4)) * KG * kWave + l;
    const int str = 64 * wave + l;  // tile row of this lane's scale word
    const uint32_t *ssrc = (const uint32_t *)((const uint8_t *)p.scales +
                                              ((size_t)g * N + subtile_row(str >> 4) + (str & 15)) * (K >> 5));
    auto dma = [&](auto stage, int kg) {
        constexpr int ST = decltype(stage)::value;
        u32x4 *A = ST == 0 ? sA0 : sA1;
        u32x4 *B = ST == 0 ? sB0 : sB1;
        uint32_t *S = ST == 0 ? sS0 : sS1;
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16(p.a + aoff[j] + (size_t)kg * 128, &A[(16 * wave + 4 * j) * 16]);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16(bsrc[j] + (size_t)kg * kWave, &B[(4 * wave + j) * kWave]);
        __builtin_amdgcn_global_load_lds(ssrc + kg, (lds_void_t *)&S[kWave * wave], 4, 0, 0);
    };

    // per-lane LDS offsets: activation chunk 4q + d of row m of the wave's
    // first m-tile (u32x4; an m-tile adds 256), the weight block of subtile
    // tsb (u32x4; subtile j adds 64 tofs(j)), the scale byte q of weight row m
    // of subtile tsb (bytes; subtile j adds 64 tofs(j))
    int a_lane[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) a_lane[d] = (64 * wm + m) * 16 + ((4 * q + d) ^ lds_swz(m));
    const int b_base = tsb * kWave + l;
    const int s_base = (16 * tsb + m) * 4 + q;
    const int mw = mrows - 64 * wm;  // rows of this wave's half that exist

    f32x4 acc[4][kFwNSW];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < kFwNSW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    dma(std::integral_constant<int, 0>(), 0);

    // step kg: stage kg % 2.  Its loads landed (this wave's: vmcnt(0); every
    // wave's: the barrier), and every wave is done with the other stage,
    // which then takes k group kg+1.  MTA of the wave's four m-tiles take
    // part (a fixed count per work item).
    auto step = [&](auto st, auto mta, int kg) {
        constexpr int S = decltype(st)::value, MTA = decltype(mta)::value;
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (kg + 1 < KG) dma(std::integral_constant<int, S ^ 1>(), kg + 1);
        if (MTA == 0) return;
        const u32x4 *A = S == 0 ? sA0 : sA1;
        const u32x4 *Bp = (S == 0 ? sB0 : sB1) + opaque_off(b_base);
        const uint8_t *Sc = (const uint8_t *)(S == 0 ? sS0 : sS1) + opaque_off(s_base);
        // the wave's weight blocks of this k group, one 16-byte read per lane
        // and subtile (a 4-byte read per k slice would take four LDS passes:
        // lanes 16 apart share a bank), and their scales (byte q of row m:
        // its 32-wide block holds every k of this lane)
        u32x4 wv[kFwNSW];
        float sc[kFwNSW];
#pragma unroll
        for (int j = 0; j < kFwNSW; ++j) {
            wv[j] = Bp[64 * tofs(j)];
            sc[j] = ue8m0_to_f32(Sc[64 * tofs(j)]);
        }
        // k slice d (32 k) at a time: the m-tiles' activation operands of
        // slice d, then per subtile its word d converted and multiplied into
        // every m-tile (each accumulator takes one instruction per slice, 32
        // independent ones in between)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const u32x4 *Ad = A + opaque_off(a_lane[d]);
            u32x4 av[MTA > 0 ? MTA : 1];
#pragma unroll
            for (int mi = 0; mi < MTA; ++mi) av[mi] = Ad[256 * mi];
#pragma unroll
            for (int j = 0; j < kFwNSW; ++j) {
                const bf16x8 bu = fp4x8_to_bf16(wv[j][d], sc[j]);
#pragma unroll
                for (int mi = 0; mi < MTA; ++mi)
                    acc[mi][j] = mfma16(__builtin_bit_cast(bf16x8, av[mi]), bu, acc[mi][j]);
            }
        }
        // keep the step's matrix instructions in the step (the instruction
        // selector otherwise moves them toward their next use, past the next
        // barrier, and two steps' operands are live at once)
#pragma unroll
        for (int mi = 0; mi < MTA; ++mi)
#pragma unroll
            for (int j = 0; j < kFwNSW; ++j) asm volatile("" : "+a"(acc[mi][j]));
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    auto kloop = [&](auto mta) {
        if constexpr (KGC != 0) {
            // unrolled whole: no loop back edge, around which the compiler
            // moves the accumulators between register files every iteration
#pragma unroll
            for (int kg = 0; kg < KGC; kg += 2) {
                step(I0(), mta, kg);
                step(I1(), mta, kg + 1);
            }
            return;
        }
        for (int kg = 0; kg < KG; kg += 2) {  // KG is even
            step(I0(), mta, kg);
            step(I1(), mta, kg + 1);
        }
    };
    if (mw > 32)
        kloop(std::integral_constant<int, 4>());
    else if (mw > 0)
        kloop(std::integral_constant<int, 2>());
    else
        kloop(std::integral_constant<int, 0>());
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load into LDS outlives the block

    // epilogue: lane (m, q) holds column m of each subtile, rows 4q..4q+3 of
    // each m-tile
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 64 * wm + 16 * mi + 4 * q + i;
            if (row >= mrows) continue;
            const bool live = srow[row] >= 0;  // a row without a source is zero
            if (ACT == MOE_ACT_SWIGLU) {
#pragma unroll
                for (int c = 0; c < kFwNSW / 2; ++c) {
                    const float gv = acc[mi][c][i], uv = acc[mi][c + kFwNSW / 2][i];
                    const float hv = silu_mul(gv, uv);
                    p.out[(size_t)(m0 + row) * (N >> 1) + subtile_row(tsb + c) + m] =
                        live ? f32_to_bf16(hv) : (uint16_t)0;
                }
            } else {
#pragma unroll
                for (int j = 0; j < kFwNSW; ++j)
                    p.out[(size_t)(m0 + row) * N + subtile_row(tsb + tofs(j)) + m] =
                        live ? f32_to_bf16(acc[mi][j][i]) : (uint16_t)0;
            }
        }
    }
}

}  // namespace

bool use_fp4_wide(const GemmArgs &p) {
    return p.fp4 && p.N % kFwTN == 0 && p.K % 256 == 0 && p.K <= 4096 && aligned(p.scales, 4);
}

void launch_fp4_wide(int act, const GemmArgs &p, hipStream_t st) {
    const int64_t max_tiles = (int64_t)p.R / kFwTM + (p.R < p.G ? p.R : p.G);
    const dim3 grid((unsigned)((max_tiles * (p.N / kFwTN) + 7) / 8 * 8));  // a whole slice per XCD
    auto go = [&](auto kgc) {
        constexpr int KGC = decltype(kgc)::value;
        if (act == MOE_ACT_SWIGLU)
            hipLaunchKernelGGL((k_mxfp4_wide<MOE_ACT_SWIGLU, KGC>), grid, dim3(512), 0, st, p);
        else
            hipLaunchKernelGGL((k_mxfp4_wide<MOE_ACT_NONE, KGC>), grid, dim3(512), 0, st, p);
    };
    if (p.K == 4096)
        go(std::integral_constant<int, 32>());
    else if (p.K == 2048)
        go(std::integral_constant<int, 16>());
    else
        go(std::integral_constant<int, 0>());
}

}  // namespace moe
