// moe_gemm_tiled.hip -- the LDS-tiled grouped W4A16 GEMM on gfx950 for
// groups with many rows (prefill, large batches), where the layer is bound by
// the matrix cores.  Compiled on its own so that its scheduling flags (all
// LDS reads of a k group issued up front) do not reach the weight-stream
// kernel, which they slow down.
//
// Method: weight-only INT4, one fp16 scale per 128 input elements, symmetric
// (model card "canada-quant/DeepSeek-V4-Flash-W4A16-FP8-MTP", "Component
// precisions"); codes unpacked with the magic-number trick and multiplied with
// bf16 activations on the matrix cores, as in moe_gemm.hip.
#include <type_traits>

#include "moe_gemm_common.h"

namespace moe {
namespace {

// One workgroup computes a TM x 128 tile (permuted rows x weight rows, TM =
// 128 or 64) of one group over the whole K with four waves (layouts at
// tiled_body).  Per 128-wide k group:
//   * the activation tile (TM gathered rows x 128 k, bf16) goes from global
//     memory straight into one of two LDS stages (global_load_lds), one k
//     group ahead, the loads spread over the step's m-tiles;
//   * each wave loads its 1 KB weight subtiles into registers two k groups
//     ahead, unpacks them once at the start of the step and reuses them for
//     its 16-row m-tiles;
//   * INT4: the -136*sum(A) term comes from the caller's row sums (or one
//     MFMA chain per m-tile without them), and the fp16 scale is applied per
//     k group in fp32 (the scales of the tile's 128 weight rows sit in LDS
//     for the whole K); FP4: the scale is folded into the conversion.
// A wave with no rows of the group skips the arithmetic, and in 64-row tiles
// a wave skips the m-tiles past the group's end.  Blocks are ordered so that
// those resident on one XCD share activation tiles and weight slices through
// its L2 (find_tile_item).
constexpr int kTN = 128;          // weight rows per tile
// sched_barrier mask: ALU, VALU, SALU, MFMA, LDS and transcendental
// instructions may be scheduled across it, global memory instructions not
constexpr int kSchedNoVmem = 0x078F;

// A wave-uniform address held as such: the loop's address arithmetic stays
// scalar, and a lane offset added to it makes the load take the scalar-base
// form (no 64-bit vector add per load)
typedef const __attribute__((address_space(1))) char *gchar_ptr;  // global memory
template <typename T>
__device__ __forceinline__ gchar_ptr uniform_ptr(const T *p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (gchar_ptr)(((uint64_t)hi << 32) | lo);
}

// dma16_untracked with the address as a scalar base plus a 32-bit lane
// offset in bytes
__device__ __forceinline__ void dma16_untracked_sv(gchar_ptr base, uint32_t voff, void *lds) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t *)lds);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(base), "s"(m0v)
        : "memory");
}
__device__ __forceinline__ void dma4_untracked_sv(gchar_ptr base, uint32_t voff, void *lds) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t *)lds);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "global_load_lds_dword %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(base), "s"(m0v)
        : "memory");
}

// the 4-byte form of dma16_untracked
__device__ __forceinline__ void dma4_untracked(const void *g, void *lds) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t *)lds);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dword %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(g), "s"(m0v)
        : "memory");
}

// Three k groups in flight through LDS.  Each stage is its own LDS variable
// and the k loop is unrolled by three so that every stage index is a
// compile-time constant: the compiler can then tell the stages apart and does
// not wait for the loads into the other stages before reading one.
// Two workgroups per CU: 72.5 KB of LDS and at most 256 registers a wave let
// two share a CU, so one computes while the other waits at its barrier or on
// its loads (with one workgroup per CU the matrix cores idled through every
// barrier, load issue and LDS read).
// SUMS: the -136*sum(A) term comes from the caller's row sums (a 4-byte load
// per row into LDS, one k group ahead like the activations) instead of an
// MFMA chain per m-tile -- a fifth of the matrix-core work, and the chain
// every m-tile's MFMAs had to wait for.
// TM: permuted rows per tile, 128 or 64 (for groups of fewer rows, where the
// second half of a 128-row tile would sit idle).
// Waves: 2 x 2 (rows x weight rows) for INT4 128-row tiles, 1 x 4 otherwise.
// A 2 x 2 wave owns 64 rows (four 16-row m-tiles) and four 16-row weight
// subtiles; a 1 x 4 wave owns every row of the tile and two subtiles, so each
// weight subtile is unpacked once per workgroup (2 x 2 unpacks it in both row
// halves; with 64-row tiles and only two m-tiles per wave the unpacking, not
// the matrix cores, would set the pace).
// A32: every byte of a lies within 2^32 of its start, so a row's offset is a
// 32-bit lane offset from a scalar base (no 64-bit vector add per load);
// otherwise 64-bit addresses (activation matrices of 4 GB and more).
template <int FMT, int ACT, bool SUMS, int TM, bool A32>
__device__ __forceinline__ void tiled_body(
    const uint16_t *__restrict__ a, const int32_t *__restrict__ gather, int n_src,
    const float *__restrict__ asums, const u32x4 *__restrict__ wq,
    const void *__restrict__ scales, const int32_t *__restrict__ offsets, int G, int R, int N,
    int K, uint16_t *__restrict__ out, int NB) {
    static_assert(FMT == kFmtInt4 || !SUMS, "row sums feed the INT4 offset term only");
    // waves along the rows: FP4 128-row tiles take 1 x 4 as well, eight
    // m-tiles per conversion of a wave's weight subtiles (prefill gate/up
    // 2307 -> 2250 us); INT4 128-row tiles lose in 1 x 4 (prefill gate/up
    // 2399 -> 2620 us even with two weight buffers and no spill)
    constexpr int WM = TM == 128 && FMT == kFmtInt4 ? 2 : 1;
    constexpr int WN = 4 / WM;             // waves along the weight rows
    constexpr int NS = 8 / WN;             // 16-row weight subtiles per wave
    constexpr int RT = TM / WM;            // rows per wave
    constexpr int MT = RT / 16;            // 16-row m-tiles per wave
    static_assert(MT == 4 || MT == 8, "a wave owns 64 or 128 rows");
    constexpr int NA = TM / 16;   // activation loads of four rows per wave and k group
    constexpr int RW = TM / 4;    // rows each wave loads
    __shared__ u32x4 sA0[TM * 16], sA1[TM * 16];
    __shared__ __attribute__((aligned(16))) float sN0[TM], sN1[TM];  // row sums, by stage
    __shared__ uint16_t sS[FMT == kFmtInt4 ? kTN * 32 : 1];  // INT4: sS[row][kg], the tile's fp16 scales
    __shared__ int srow[TM];
    // the wave index is uniform: LDS addresses derived from it stay scalar
    // (M0 of the loads into LDS without a readfirstlane per load)
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), l = lane_id();
    const int m = l & 15, q = l >> 4;
    const int wm = WM == 2 ? wave >> 1 : 0, wn = WM == 2 ? wave & 1 : wave;
    TileItem it;
    if (!workgroup_tile_item(NB, TM, offsets, G, R, it)) return;  // the whole workgroup: no work item
    const int g = it.g, m0 = it.m0, mrows = it.mrows, nb = it.nb;
    const int KG = K >> 7, NT = N >> 4;

    // weight row of subtile t (0..7) of the tile; wave wn owns t = NS*wn + s.
    // SwiGLU: a wave's first NS/2 subtiles are gate rows, the others the up
    // rows of the same columns
    auto subtile_row = [&](int t) {
        if (ACT == MOE_ACT_SWIGLU) {
            constexpr int H2 = NS / 2;
            const int w = t / NS, s = t - w * NS;
            const int c = nb * 64 + 16 * H2 * w + 16 * (s % H2);
            return s >= H2 ? (N >> 1) + c : c;
        }
        return nb * kTN + 16 * t;
    };
    const u32x4 *wg = wq + (size_t)g * NT * KG * kWave;
    const uint16_t *sg = (const uint16_t *)scales + (size_t)g * N * KG;         // INT4: fp16 [N][KG]
    const uint8_t *sg8 = (const uint8_t *)scales + (size_t)g * N * (K >> 5);   // FP4: UE8M0 [N][K/32]

    if (tid < TM) {
        int sr = -1;
        if (tid < mrows) {
            if (gather) {
                const int t = gather[m0 + tid];
                sr = (unsigned)t < (unsigned)n_src ? t : -1;
            } else {
                sr = m0 + tid;
            }
        }
        srow[tid] = sr;
    }
    if constexpr (FMT == kFmtInt4) {
        // sS[j][kg] for tile row j: subtile t's 16 rows are consecutive rows
        // of the [N][KG] scales, 32*KG contiguous bytes, which go straight
        // into LDS (wave w moves subtiles 2w and 2w+1; read in the first
        // step, after its wait and barrier).  Scales only 2-byte aligned
        // take the register path.
        if ((reinterpret_cast<uintptr_t>(sg) & 3) == 0) {
            const int nd = 8 * KG;  // dwords per subtile
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int t = 2 * wave + h;
                const uint32_t *src = reinterpret_cast<const uint32_t *>(sg + (size_t)subtile_row(t) * KG);
                uint32_t *dst = reinterpret_cast<uint32_t *>(sS) + t * nd;
                for (int c = 0; c < nd; c += kWave)
                    if (c + l < nd) __builtin_amdgcn_global_load_lds(src + c + l, (lds_void_t *)(dst + c), 4, 0, 0);
            }
        } else {
            for (int i = tid; i < kTN * KG; i += 256) {
                const int j = i / KG, kg = i - j * KG;
                sS[i] = sg[(size_t)(subtile_row(j >> 4) + (j & 15)) * KG + kg];
            }
        }
    }
    __syncthreads();

    // activation loads: wave w moves rows RW*w .. RW*w+RW-1, NA loads of four
    // rows (rows without a source read row 0 and are never stored)
    // element offsets (64-bit: rows x K of a can pass 2^32 elements, the
    // down projection of 300K tokens), or byte offsets when A32
    size_t aoff[NA];
    uint32_t aoffb[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) {
        const int r = RW * wave + 4 * j + (l >> 4);
        const int c = (l & 15) ^ lds_swz(r);
        if constexpr (A32)
            aoffb[j] = ((uint32_t)max(srow[r], 0) * (uint32_t)K + 8u * (uint32_t)c) * 2u;
        else
            aoff[j] = (size_t)max(srow[r], 0) * K + 8 * c;
    }
    // row sums: lanes 0..RW-1 of wave w load those of its rows
    const uint32_t soff = (uint32_t)max(srow[RW * wave + (l & (RW - 1))], 0) * (uint32_t)KG;
    auto dma_a = [&](auto stage, int kg, auto tracked, int p) {  // part p of 4: loads [p*NA/4, (p+1)*NA/4)
        u32x4 *A = decltype(stage)::value == 0 ? sA0 : sA1;
        if (SUMS && p == 0 && l < RW) {
            float *S = decltype(stage)::value == 0 ? sN0 : sN1;
            if constexpr (A32) {  // (the step's explicit wait and barrier cover it)
                dma4_untracked_sv(uniform_ptr(asums + kg), 4u * soff, &S[RW * wave]);
            } else {
                const float *src = asums + (size_t)soff + kg;
                if (decltype(tracked)::value)
                    __builtin_amdgcn_global_load_lds(src, (lds_void_t *)&S[RW * wave], 4, 0, 0);
                else
                    dma4_untracked(src, &S[RW * wave]);
            }
        }
        const gchar_ptr abase = uniform_ptr(a + (size_t)kg * 128);
#pragma unroll
        for (int j = p * NA / 4; j < (p + 1) * NA / 4; ++j) {
            void *dst = &A[(RW * wave + 4 * j) * 16];
            if constexpr (A32) {
                // written as assembly: the compiler's form of the load keeps
                // a 64-bit vector address (it hoists the offset's extension
                // out of the loop); the step's explicit wait and barrier
                // cover it either way
                dma16_untracked_sv(abase, aoffb[j], dst);
            } else {
                const uint16_t *src = a + aoff[j] + (size_t)kg * 128;
                if (decltype(tracked)::value)
                    dma16(src, dst);
                else
                    dma16_untracked(src, dst);
            }
        }
    };
    // this wave's weight subtiles t = NS*wn + s
    // (FP4: and their scale bytes -- row subtile_row + m, the 32-wide block q
    // of each k group -- loaded with the weights, one k group per load_b)
    // Addresses as a wave-uniform base plus a 32-bit lane offset, the form
    // the loads take with the base in scalar registers (no 64-bit vector
    // address arithmetic per load)
    const u32x4 *bsrc[NS];    // subtile bases
    const uint8_t *ssrc[NS];  // FP4: the subtile's scale rows
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        bsrc[s] = wg + (size_t)(subtile_row(NS * wn + s) >> 4) * KG * kWave;
        ssrc[s] = sg8 + (size_t)subtile_row(NS * wn + s) * (K >> 5);
    }
    const uint32_t boff = 16u * (uint32_t)l;                       // bytes
    const uint32_t soffb = (uint32_t)m * (uint32_t)(K >> 5) + (uint32_t)q;  // bytes
    constexpr int NLB = FMT == kFmtInt4 ? NS : 2 * NS;  // loads of one load_b
    auto load_b = [&](int kg, u32x4 *br, uint32_t *bs) {
#pragma unroll
        for (int s = 0; s < NS; ++s) br[s] = *(const __attribute__((address_space(1))) u32x4 *)(uniform_ptr(bsrc[s] + (size_t)kg * kWave) + boff);
        if constexpr (FMT == kFmtFp4) {
#pragma unroll
            for (int s = 0; s < NS; ++s) bs[s] = *(const __attribute__((address_space(1))) uint8_t *)(uniform_ptr(ssrc[s] + kg * 4) + soffb);
        }
    };

    bf16x8 bneg;
#pragma unroll
    for (int i = 0; i < 8; ++i) bneg[i] = __builtin_bit_cast(__bf16, kNeg136);
    f32x4 acc[MT][NS];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[i][s] = f32x4{0.f, 0.f, 0.f, 0.f};
    // weight register buffers: a step unpacks its buffer at its start, so
    // two give the loads of k group kg+2 the whole step kg+1 as lead.  The
    // INT4 128-row instance keeps three (prefill gate/up 2399 against 2436
    // us with two; stack43 gate/up 840 -> 832 us and FP4 prefill 2307 ->
    // 2257 us with two)
    constexpr int NBUF = FMT == kFmtInt4 && TM == 128 ? 3 : 2;
    u32x4 braw[NBUF][NS];
    uint32_t bsc[NBUF][NS];  // FP4 scale bytes

    // in flight before the loop: activations of k group 0 (LDS stage 0),
    // weights of k groups 0 and 1 (register buffers 0 and 1)
#pragma unroll
    for (int p = 0; p < 4; ++p) dma_a(std::integral_constant<int, 0>(), 0, std::false_type(), p);
    load_b(0, braw[0], bsc[0]);
    load_b(min(1, KG - 1), braw[1], bsc[1]);

    // step kg: activations in LDS stage kg % 2, weights in buffer kg % NBUF;
    // it issues the activations of kg+1 (spread over its m-tiles) and, last,
    // the weights of kg+2 (into buffer (kg+2) % NBUF: with two, the one it
    // unpacked at its start) -- the weights come from HBM and need the
    // longer lead.  Past the end the loads repeat the last k group (never
    // read).
    // MTA: the m-tiles this wave multiplies in every step of the work item
    // (0: loads only), fixed per k loop so that no accumulator crosses a
    // branch inside it (a skipped m-tile's accumulators otherwise cost a
    // register copy each per step).  -1: all MT, and a wave without rows
    // branches to the loads in every step (128-row tiles: without that
    // branch, which bounds the scheduling region, the compiler moves work
    // across steps and spills)
    auto step = [&](auto stage, auto wbuf, auto mta, int kg) {
        constexpr int ST = decltype(stage)::value, WB = decltype(wbuf)::value;
        constexpr int MTA = decltype(mta)::value < 0 ? MT : decltype(mta)::value;
        constexpr int SN = ST ^ 1;  // the stage loaded in this step
        const u32x4 *A = ST == 0 ? sA0 : sA1;
        const float *S = ST == 0 ? sN0 : sN1;
        // every load of this wave but the last NLB (the weights of kg+1)
        // has landed: the activations of kg in LDS, its weights in
        // registers; after the barrier every wave's have, and every wave is
        // done with the other stage
        __builtin_amdgcn_s_waitcnt(0x0F70 | NLB);  // vmcnt(NLB)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        const int ka = min(kg + 1, KG - 1), kb = min(kg + 2, KG - 1);
        // The weights of kg+2 are this step's last NLB loads: the next step
        // waits until at most NLB are outstanding and then reads the stage
        // the other waves loaded, so every load into LDS goes first (a
        // scheduling barrier that only arithmetic and LDS instructions may
        // cross keeps the compiler from moving one past them)
        if (MTA == 0 || (decltype(mta)::value < 0 && mrows - RT * wm <= 0)) {  // no rows: loads only
#pragma unroll
            for (int p = 0; p < 4; ++p) dma_a(std::integral_constant<int, SN>(), ka, std::true_type(), p);
            __builtin_amdgcn_sched_barrier(kSchedNoVmem);
            load_b(kb, braw[(WB + 2) % NBUF], bsc[(WB + 2) % NBUF]);
            return;
        }
        bf16x8 bu[NS][4];
        float sc[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if constexpr (FMT == kFmtInt4) {
#pragma unroll
                for (int d = 0; d < 4; ++d) bu[s][d] = unpack_codes(braw[WB][s][d]);
                sc[s] = half_bits_to_f32(sS[(16 * (NS * wn + s) + m) * KG + kg]);
            } else {
                const float e = ue8m0_to_f32(bsc[WB][s]);
#pragma unroll
                for (int d = 0; d < 4; ++d) bu[s][d] = fp4x8_to_bf16(braw[WB][s][d], e);
            }
        }
        // PIPE (INT4 128-row tiles): the activations and row sums of m-tile
        // mi+1 are read from LDS once m-tile mi's MFMAs are issued, so their
        // latency passes during mi's scale FMAs instead of ahead of mi+1's
        // MFMAs (in 64-row tiles the extra registers spill)
        constexpr bool PIPE = FMT == kFmtInt4 && TM == 128;
        u32x4 av[4];
        f32x4 sv;
        auto read_a = [&](int mi) {
            const int r = RT * wm + 16 * mi + m;
#pragma unroll
            for (int d = 0; d < 4; ++d) av[d] = A[r * 16 + ((4 * q + d) ^ lds_swz(r))];
            // rows 4q..4q+3 of the m-tile, this lane's accumulator rows
            if constexpr (SUMS) sv = *(const f32x4 *)&S[RT * wm + 16 * mi + 4 * q];
        };
        if constexpr (PIPE) read_a(0);
#pragma unroll
        for (int mi = 0; mi < MTA; ++mi) {
#pragma unroll
            for (int p = mi * 4 / MT; p < (mi + 1) * 4 / MT; ++p)
                dma_a(std::integral_constant<int, SN>(), ka, std::true_type(), p);
            if constexpr (!PIPE) read_a(mi);
            if constexpr (FMT == kFmtFp4) {
#pragma unroll
                for (int d = 0; d < 4; ++d)
#pragma unroll
                    for (int s = 0; s < NS; ++s)
                        acc[mi][s] = mfma16(__builtin_bit_cast(bf16x8, av[d]), bu[s][d], acc[mi][s]);
                continue;
            }
            f32x4 nc = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (SUMS) {
                nc = sv * -136.0f;
            } else {
#pragma unroll
                for (int d = 0; d < 4; ++d) nc = mfma16(__builtin_bit_cast(bf16x8, av[d]), bneg, nc);
            }
            f32x4 t[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) t[s] = nc;
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
                for (int s = 0; s < NS; ++s) t[s] = mfma16(__builtin_bit_cast(bf16x8, av[d]), bu[s][d], t[s]);
            if (PIPE && mi + 1 < MTA) read_a(mi + 1);
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mi][s][i] = __builtin_fmaf(sc[s], t[s][i], acc[mi][s][i]);
            // PIPE: the next m-tile's first use of its reads stays behind
            // these FMAs (the compiler would hoist its row-sum products, and
            // the wait for the reads with them, right after the reads).
            // Otherwise no scheduling barrier between m-tiles: the next
            // m-tile's LDS reads move up over this one's MFMAs and scale FMAs
            // (stack43 gate/up 932 -> 880 us; a few registers of the 64-row
            // instances spill); with eight m-tiles, every second one, which
            // bounds the hoisted reads
            if (PIPE || (MT == 8 && (mi & 1))) __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int p = MTA * 4 / MT; p < 4; ++p)  // the activation loads of the m-tiles past MTA
            dma_a(std::integral_constant<int, SN>(), ka, std::true_type(), p);
        __builtin_amdgcn_sched_barrier(kSchedNoVmem);
        load_b(kb, braw[(WB + 2) % NBUF], bsc[(WB + 2) % NBUF]);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    auto kloop = [&](auto mta) {
        if constexpr (NBUF == 2) {
            for (int kg = 0; kg < KG; kg += 2) {  // (stage, buffer) cycles with period 2
                step(I0(), I0(), mta, kg);
                if (kg + 1 >= KG) break;
                step(I1(), I1(), mta, kg + 1);
            }
        } else {
            using I2 = std::integral_constant<int, 2>;
            for (int kg = 0; kg < KG; kg += 6) {  // (stage, buffer) cycles with period 6
                step(I0(), I0(), mta, kg);
                if (kg + 1 >= KG) break;
                step(I1(), I1(), mta, kg + 1);
                if (kg + 2 >= KG) break;
                step(I0(), I2(), mta, kg + 2);
                if (kg + 3 >= KG) break;
                step(I1(), I0(), mta, kg + 3);
                if (kg + 4 >= KG) break;
                step(I0(), I1(), mta, kg + 4);
                if (kg + 5 >= KG) break;
                step(I1(), I2(), mta, kg + 5);
            }
        }
    };
    // 64-row tiles multiply only the m-tiles that hold rows; 128-row tiles
    // all of a wave's four (there skipping cost more than it saved), and a
    // wave of the lower half without rows only loads
    if constexpr (TM != 64) {
        kloop(std::integral_constant<int, -1>());
    } else {
        // one row of waves: every wave has the tile's mrows >= 1 rows, so
        // there is no loads-only loop (in one, the compiler drops the weight
        // loads nothing reads, and the step's wait would then let loads into
        // LDS stay outstanding past the barrier)
        const int mta = min(MT, (mrows + 15) >> 4);
        if (mta == 1)
            kloop(std::integral_constant<int, 1>());
        else if (mta == 2)
            kloop(std::integral_constant<int, 2>());
        else if (mta == 3)
            kloop(std::integral_constant<int, 3>());
        else
            kloop(std::integral_constant<int, MT>());
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load into LDS outlives the block

    int nrow[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) nrow[s] = subtile_row(NS * wn + s);
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = RT * wm + 16 * mi + 4 * q + i;
            if (row >= mrows) continue;
            const bool live = srow[row] >= 0;  // a row without a source is zero
            uint16_t *orow = out + (size_t)(m0 + row) * (ACT == MOE_ACT_SWIGLU ? (N >> 1) : N);
            if (ACT == MOE_ACT_SWIGLU) {
#pragma unroll
                for (int s = 0; s < NS / 2; ++s) {
                    const float gv = acc[mi][s][i], uv = acc[mi][s + NS / 2][i];
                    const float hv = silu_mul(gv, uv);
                    orow[nrow[s] + m] = live ? f32_to_bf16(hv) : (uint16_t)0;
                }
            } else {
#pragma unroll
                for (int s = 0; s < NS; ++s) orow[nrow[s] + m] = live ? f32_to_bf16(acc[mi][s][i]) : (uint16_t)0;
            }
        }
    }
}

#define MOE_TILED_ARGS                                                                           \
    const uint16_t *__restrict__ a, const int32_t *__restrict__ gather, int n_src,                \
        const float *__restrict__ asums, const u32x4 *__restrict__ wq,                            \
        const void *__restrict__ scales, const int32_t *__restrict__ offsets, int G, int R, int N, \
        int K, uint16_t *__restrict__ out, int NB
#define MOE_TILED_PASS a, gather, n_src, asums, wq, scales, offsets, G, R, N, K, out, NB

template <int ACT, bool SUMS, int TM, bool A32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TM == 64 ? 3 : 2, TM == 64 ? 3 : 2))) void
k_w4a16_tiled(MOE_TILED_ARGS) {
    tiled_body<kFmtInt4, ACT, SUMS, TM, A32>(MOE_TILED_PASS);
}

template <int ACT, int TM, bool A32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TM == 64 ? 3 : 2, TM == 64 ? 3 : 2))) void
k_mxfp4_tiled(MOE_TILED_ARGS) {
    tiled_body<kFmtFp4, ACT, false, TM, A32>(MOE_TILED_PASS);
}

}  // namespace

bool use_tiled(int T, int N, int K) {
    return T >= MOE_TILED_MIN_TOKENS && N % kTN == 0 && K <= 4096;
}

template <int TM, bool A32>
void launch_tiled_tm(int act, bool fp4, const GemmArgs &p, hipStream_t st) {
    const int NB = p.N / kTN;
    const int64_t max_tiles = (int64_t)p.R / TM + (p.R < p.G ? p.R : p.G);
    const int64_t blocks = (max_tiles * NB + 7) / 8 * 8;  // a whole slice per XCD
    auto kern = fp4 ? (act == MOE_ACT_SWIGLU ? k_mxfp4_tiled<MOE_ACT_SWIGLU, TM, A32> : k_mxfp4_tiled<MOE_ACT_NONE, TM, A32>)
                : act == MOE_ACT_SWIGLU
                    ? (p.sums ? k_w4a16_tiled<MOE_ACT_SWIGLU, true, TM, A32> : k_w4a16_tiled<MOE_ACT_SWIGLU, false, TM, A32>)
                    : (p.sums ? k_w4a16_tiled<MOE_ACT_NONE, true, TM, A32> : k_w4a16_tiled<MOE_ACT_NONE, false, TM, A32>);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, st, p.a, p.gather, p.n_src,
                       fp4 ? nullptr : p.sums, p.wq, p.scales, p.offsets, p.G, p.R, p.N, p.K, p.out, NB);
}

// 64-row tiles when the groups average fewer than 96 rows (a 128-row tile
// would leave half its waves idle), 128-row tiles otherwise (the activation
// tile in LDS then feeds twice the weight columns per byte read).
void launch_tiled(int act, const GemmArgs &p, hipStream_t st, bool fp4) {
    if (fp4 && use_fp4_wide(p)) {
        launch_fp4_wide(act, p, st);
        return;
    }
    // byte offsets into a fit 32 bits (a's rows: the gathered source's, or R)
    const bool a32 = (int64_t)(p.gather ? p.n_src : p.R) * p.K * 2 <= (int64_t)0xFFFFFFFF;
    if ((int64_t)p.R < 96 * (int64_t)p.G) {
        if (a32)
            launch_tiled_tm<64, true>(act, fp4, p, st);
        else
            launch_tiled_tm<64, false>(act, fp4, p, st);
    } else {
        if (a32)
            launch_tiled_tm<128, true>(act, fp4, p, st);
        else
            launch_tiled_tm<128, false>(act, fp4, p, st);
    }
}

}  // namespace moe
