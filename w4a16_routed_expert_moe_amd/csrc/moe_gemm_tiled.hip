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

// One workgroup computes a 128 x 128 tile (permuted rows x weight rows) of
// one group over the whole K, four waves in a 2 x 2 layout of 64 x 64.  Per
// 128-wide k group:
//   * the activation tile (128 gathered rows x 128 k, bf16, 32 KB) and the
//     eight 1 KB weight subtiles go from global memory straight into LDS
//     (global_load_lds), three k groups in flight;
//   * each wave unpacks its four weight subtiles once and reuses them for its
//     four 16-row m-tiles; the -136*sum(A) term is one MFMA chain per m-tile,
//     shared by the four n-tiles; the fp16 scale is applied per k group in
//     fp32 (scales of the tile's 128 weight rows sit in LDS for the whole K).
// A wave whose 64 rows all lie past the group's end skips the arithmetic.
// Blocks are ordered so that those resident on one XCD share activation
// tiles and weight slices through its L2 (find_item_tiled).
constexpr int kTM = 128;          // permuted rows per tile
constexpr int kTN = 128;          // weight rows per tile

__device__ __forceinline__ bool find_item_tiled(int b, int NB, const int32_t *__restrict__ offsets,
                                                int G, int &g_out, int &m0, int &mrows, int &nb) {
    // The work list: groups in order; a group's m-tiles in chunks of up to
    // four; inside a chunk n-block-major, so 32 consecutive items cover 8
    // n-blocks x 4 m-tiles.  Blocks are dealt to the eight XCDs in turn
    // (block b runs on XCD b % 8) and XCD x takes the contiguous slice
    // [x*per, (x+1)*per) of the list, so the blocks resident on one XCD at a
    // time share activation tiles and weight slices in that XCD's L2.
    const int l = lane_id();
    int total = 0;
    for (int g0 = 0; g0 < G; g0 += kWave) {
        const int g = g0 + l;
        const int n = g < G ? offsets[g + 1] - offsets[g] : 0;
        const int items = (n > 0 ? (n + kTM - 1) / kTM : 0) * NB;
        total += __shfl(wave_incl_scan(items), kWave - 1, kWave);
    }
    const int per = (total + 7) >> 3;
    const int x = b & 7, j = b >> 3;
    const int item = x * per + j;
    if (j >= per || item >= total) return false;
    int before = 0;
    for (int g0 = 0; g0 < G; g0 += kWave) {
        const int g = g0 + l;
        int n = 0, lo = 0;
        if (g < G) {
            lo = offsets[g];
            n = offsets[g + 1] - lo;
        }
        const int mt = n > 0 ? (n + kTM - 1) / kTM : 0;
        const int items = mt * NB;
        const int incl = wave_incl_scan(items);
        const int tot = __shfl(incl, kWave - 1, kWave);
        if (item < before + tot) {
            const bool mine = g < G && item >= before + incl - items && item < before + incl;
            const int src = __ffsll((unsigned long long)__ballot(mine)) - 1;
            const int local = item - before - (__shfl(incl, src, kWave) - __shfl(items, src, kWave));
            const int mt_s = __shfl(mt, src, kWave);
            const int c = local / (4 * NB), rem = local - c * 4 * NB;
            const int mc = min(4, mt_s - 4 * c);
            const int nbi = rem / mc;
            const int mi = 4 * c + rem - nbi * mc;
            g_out = g0 + src;
            m0 = __shfl(lo, src, kWave) + mi * kTM;
            mrows = min(kTM, __shfl(n, src, kWave) - mi * kTM);
            nb = nbi;
            return true;
        }
        before += tot;
    }
    return false;
}

typedef __attribute__((address_space(3))) void lds_void_t;

// 16 bytes per lane straight from global memory into LDS: lane l's bytes land
// at lds + 16*l (the LDS address is wave-uniform); counted by vmcnt.
__device__ __forceinline__ void dma16(const void *g, void *lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void_t *)lds, 16, 0, 0);
}
// The same load written as inline assembly, which the compiler's wait-count
// pass does not track.  Used for the loads issued ahead of the pipelined k
// loop: tracked there, they make the pass wait for every load into LDS
// before the loop's first LDS read.  Their completion is ordered by the
// loop's own explicit wait and barrier.
// M0 is a reserved register, so the assembly restores it: to the compiler
// it is unchanged.
__device__ __forceinline__ void dma16_untracked(const void *g, void *lds) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t *)lds);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(g), "s"(m0v)
        : "memory");
}

// Three k groups in flight through LDS.  Each stage is its own LDS variable
// and the k loop is unrolled by three so that every stage index is a
// compile-time constant: the compiler can then tell the stages apart and does
// not wait for the loads into the other stages before reading one.
template <int ACT>
__global__ __launch_bounds__(256) void k_w4a16_tiled(
    const uint16_t *__restrict__ a, const int32_t *__restrict__ gather, int n_src,
    const u32x4 *__restrict__ wq, const uint16_t *__restrict__ scales,
    const int32_t *__restrict__ offsets, int G, int R, int N, int K, uint16_t *__restrict__ out,
    int NB) {
    // activation stage: [row][16 chunks of 16 B], chunk c of row r at slot
    // c ^ (r & 15) so that the 16 rows one MFMA operand read touches fall in
    // distinct banks; weight stage: [8 subtiles][1 KB], the prepacked blocks
    // as they are in memory; scales: [K/128][128 weight rows]
    __shared__ u32x4 sA0[kTM * 16], sA1[kTM * 16], sA2[kTM * 16];
    __shared__ u32x4 sB0[8 * kWave], sB1[8 * kWave], sB2[8 * kWave];
    __shared__ uint16_t sS[kTN * 32];
    __shared__ int srow[kTM];
    const int tid = threadIdx.x, wave = tid >> 6, l = lane_id();
    const int m = l & 15, q = l >> 4;
    const int wm = wave >> 1, wn = wave & 1;
    int g, m0, mrows, nb;
    if (!find_item_tiled(blockIdx.x, NB, offsets, G, g, m0, mrows, nb)) return;  // uniform
    if (m0 < 0 || m0 >= R) return;
    g = __builtin_amdgcn_readfirstlane(g);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    nb = __builtin_amdgcn_readfirstlane(nb);
    mrows = __builtin_amdgcn_readfirstlane(min(mrows, R - m0));
    const int KG = K >> 7, NT = N >> 4;

    // weight rows of the block's 8 subtiles: subtile t = 4*wn + s belongs to
    // wave column wn; for SwiGLU s = 0,1 are gate rows and s = 2,3 the
    // matching up rows
    auto subtile_row = [&](int t) {
        if (ACT == MOE_ACT_SWIGLU) {
            const int c = nb * 64 + 32 * (t >> 2) + 16 * (t & 1);
            return (t & 2) ? (N >> 1) + c : c;
        }
        return nb * kTN + 16 * t;
    };
    const u32x4 *wg = wq + (size_t)g * NT * KG * kWave;
    const uint16_t *sg = scales + (size_t)g * N * KG;

    if (tid < kTM) {
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
    for (int i = tid; i < kTN * KG; i += 256) {  // sS[kg][row]: a lane's 16 rows are adjacent
        const int j = i & (kTN - 1), kg = i >> 7;
        sS[i] = sg[(size_t)(subtile_row(j >> 4) + (j & 15)) * KG + kg];
    }
    __syncthreads();

    // load plan: wave w moves activation rows 32w..32w+31 (8 loads of 4 rows;
    // rows without a source read row 0 and are never stored) and weight
    // subtiles 2w, 2w+1 of every k group: 10 loads per wave and k group
    const uint16_t *arow_ptr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = 32 * wave + 4 * j + (l >> 4);
        const int c = (l & 15) ^ (r & 15);
        arow_ptr[j] = a + (size_t)max(srow[r], 0) * K + 8 * c;
    }
    const u32x4 *bsrc0 = wg + (size_t)(subtile_row(2 * wave) >> 4) * KG * kWave + l;
    const u32x4 *bsrc1 = wg + (size_t)(subtile_row(2 * wave + 1) >> 4) * KG * kWave + l;
    // the loads of one k group into one stage, in four parts
    auto loads = [&](auto stage, int kg, auto tracked) {
        constexpr int ST = decltype(stage)::value;
        u32x4 *A = ST == 0 ? sA0 : ST == 1 ? sA1 : sA2;
        u32x4 *B = ST == 0 ? sB0 : ST == 1 ? sB1 : sB2;
        auto ld = [](const void *g, void *lds) {
            if (decltype(tracked)::value)
                dma16(g, lds);
            else
                dma16_untracked(g, lds);
        };
        // part p of the k group's ten loads: p = 0 the two weight blocks and
        // activation load 0, p = 1 loads 1-2, p = 2 loads 3-5, p = 3 loads 6-7
        auto part = [=](int p) {  // by value: it outlives this call
            if (p == 0) {
                ld(bsrc0 + (size_t)kg * kWave, &B[(2 * wave) * kWave]);
                ld(bsrc1 + (size_t)kg * kWave, &B[(2 * wave + 1) * kWave]);
            }
            const int j0 = p == 0 ? 0 : p == 1 ? 1 : p == 2 ? 3 : 6;
            const int j1 = p == 0 ? 1 : p == 1 ? 3 : p == 2 ? 6 : 8;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (j >= j0 && j < j1) ld(arow_ptr[j] + kg * 128, &A[(32 * wave + 4 * j) * 16]);
        };
        return part;
    };
    auto issue = [&](auto stage, int kg, auto tracked) {
        auto part = loads(stage, kg, tracked);
#pragma unroll
        for (int p = 0; p < 4; ++p) part(p);
    };

    bf16x8 bneg;
#pragma unroll
    for (int i = 0; i < 8; ++i) bneg[i] = __builtin_bit_cast(__bf16, kNeg136);
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[i][s] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto step = [&](auto stage, int kg) {
        constexpr int ST = decltype(stage)::value;
        const u32x4 *A = ST == 0 ? sA0 : ST == 1 ? sA1 : sA2;
        const u32x4 *B = ST == 0 ? sB0 : ST == 1 ? sB1 : sB2;
        // this wave's loads for kg have landed once at most the next k
        // group's 10 are outstanding; after the barrier every wave's have,
        // and every wave is done reading the stage the next issue refills.
        // Every step issues exactly 10 loads (past the last k group it
        // reloads the last one into a stage nobody reads) so that the wait
        // count is the same on every path.
        __builtin_amdgcn_s_waitcnt(0x0F7A);  // vmcnt(10)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // The loads for k group kg+2 go out in four parts, one ahead of each
        // m-tile's MFMAs: a CU's vector memory path takes about 64 bytes a
        // clock, so the 40 KB of a k group issued at once would stall every
        // wave here instead of running beside the matrix cores.
        auto next = loads(std::integral_constant<int, (ST + 2) % 3>(), min(kg + 2, KG - 1),
                          std::true_type());

        // A wave whose 64 rows are all past the group's end issues its loads
        // and skips the arithmetic; otherwise the step is straight-line code
        // (rows past the end compute values that are never stored) so that
        // the scheduler can overlap one m-tile's scale FMAs and the next
        // m-tile's LDS reads with the current m-tile's MFMAs.
        if (64 * wm >= mrows) {
#pragma unroll
            for (int p = 0; p < 4; ++p) next(p);
            return;
        }
        bf16x8 bu[4][4];
        float sc[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int t = 4 * wn + s;
            const u32x4 w = B[t * kWave + l];
#pragma unroll
            for (int d = 0; d < 4; ++d) bu[s][d] = unpack_codes(w[d]);
            sc[s] = half_bits_to_f32(sS[kg * kTN + 16 * t + m]);
        }
        auto load_a = [&](int mi, u32x4 *av) {
            const int r = 64 * wm + 16 * mi + m;
#pragma unroll
            for (int d = 0; d < 4; ++d) av[d] = A[r * 16 + ((4 * q + d) ^ (r & 15))];
        };
        auto apply_scales = [&](int mi, const f32x4 *t) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mi][s][i] = __builtin_fmaf(sc[s], t[s][i], acc[mi][s][i]);
        };
        u32x4 av[2][4];
        f32x4 tp[4];
        load_a(0, av[0]);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            next(mi);
            if (mi < 3) load_a(mi + 1, av[(mi + 1) & 1]);
            const u32x4 *a4 = av[mi & 1];
            f32x4 nc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int d = 0; d < 4; ++d) nc = mfma16(__builtin_bit_cast(bf16x8, a4[d]), bneg, nc);
            f32x4 t[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) t[s] = nc;
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    t[s] = mfma16(__builtin_bit_cast(bf16x8, a4[d]), bu[s][d], t[s]);
            if (mi > 0) apply_scales(mi - 1, tp);
#pragma unroll
            for (int s = 0; s < 4; ++s) tp[s] = t[s];
            __builtin_amdgcn_sched_barrier(0);
        }
        apply_scales(3, tp);
    };

    issue(std::integral_constant<int, 0>(), 0, std::false_type());
    issue(std::integral_constant<int, 1>(), min(1, KG - 1), std::false_type());
    for (int kg = 0; kg < KG; kg += 3) {
        step(std::integral_constant<int, 0>(), kg);
        if (kg + 1 >= KG) break;
        step(std::integral_constant<int, 1>(), kg + 1);
        if (kg + 2 >= KG) break;
        step(std::integral_constant<int, 2>(), kg + 2);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load into LDS outlives the block

    int nrow[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) nrow[s] = subtile_row(4 * wn + s);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 64 * wm + 16 * mi + 4 * q + i;
            if (row >= mrows) continue;
            const bool live = srow[row] >= 0;  // a row without a source is zero
            uint16_t *orow = out + (size_t)(m0 + row) * (ACT == MOE_ACT_SWIGLU ? (N >> 1) : N);
            if (ACT == MOE_ACT_SWIGLU) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const float gv = acc[mi][s][i], uv = acc[mi][s + 2][i];
                    const float hv = gv * uv * __frcp_rn(1.0f + __expf(-gv));
                    orow[nrow[s] + m] = live ? f32_to_bf16(hv) : (uint16_t)0;
                }
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) orow[nrow[s] + m] = live ? f32_to_bf16(acc[mi][s][i]) : (uint16_t)0;
            }
        }
    }
}

// Large groups take the tiled kernel: from 256 tokens on the average group
// fills most of a 128-row tile; below, the weight stream wins.
}  // namespace

bool use_tiled(int T, int N, int K) { return T >= 256 && N % kTN == 0 && K <= 4096; }

void launch_tiled(int act, const GemmArgs &p, hipStream_t st) {
    const int NB = p.N / kTN;
    const int64_t max_tiles = (int64_t)p.R / kTM + (p.R < p.G ? p.R : p.G);
    const int64_t blocks = (max_tiles * NB + 7) / 8 * 8;  // a whole slice per XCD
    auto kern = act == MOE_ACT_SWIGLU ? k_w4a16_tiled<MOE_ACT_SWIGLU> : k_w4a16_tiled<MOE_ACT_NONE>;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, st, p.a, p.gather, p.n_src, p.wq,
                       p.scales, p.offsets, p.G, p.R, p.N, p.K, p.out, NB);
}

}  // namespace moe
