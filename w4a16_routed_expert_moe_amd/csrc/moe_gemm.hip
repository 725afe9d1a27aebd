// moe_gemm.hip -- grouped W4A16 GEMM of the expert projections on gfx950.
//
// Method: weight-only INT4 (one fp16 scale per 128 input elements, symmetric;
// model card "canada-quant/DeepSeek-V4-Flash-W4A16-FP8-MTP", "Component
// precisions"), dequantised in registers and multiplied with bf16
// activations on the matrix cores -- the scheme the Marlin kernel applies on
// Hopper ("Throughputmaxxing: DeepSeek-V4-Flash on Isambard-AI", "A pass through
// the model"), redesigned here for CDNA4.
//
// Weight-stream kernel (k_w4a16_stream), the path for small groups, where the
// layer is bound by HBM weight traffic.  One workgroup owns an n-block of
// 16*NSUB weight rows (for SwiGLU half gate rows and the matching up rows) and
// at most ROWS permuted rows of one group; its waves split K and add their
// partial tiles through LDS at the end.
//   * B operand (weights): each lane reads 16 bytes of a 1 KB block of the
//     prepacked layout, so a wave load is one contiguous 1 KB stream; the
//     codes go straight from HBM to registers (no LDS).
//   * Unpack: a code u = q+8 placed under the bf16 exponent of 128 gives the
//     exact bf16 value 128+u with one AND-OR per pair of codes.  The MFMA
//     then yields sum A*(q+136); the -136*sum(A) term is one extra MFMA
//     chain per k group with a constant -136 B operand, shared by all
//     subtiles, and is fed in as the accumulator input.
//   * Scales: acc += s[n][kg] * tile after each 128-wide k group (fp32).
//   * A operand (activations): each wave stages the rows x its k slice in its
//     own LDS region, bf16 in natural k order.
// v_mfma_f32_16x16x32_bf16: A = 16 rows x 32 k (lane l: row l%16, k slots
// 8*(l/16)..+8), B = 32 k x 16 cols (lane l: col l%16), D = 16x16 fp32 with
// lane l holding rows 4*(l/16)..+4 of column l%16.  Here rows are permuted
// token rows and columns are weight rows.
#include <type_traits>

#include "moe_common.h"

namespace moe {
namespace {

constexpr uint32_t kMagic = 0x43004300u;  // bf16 128.0 in both halves
constexpr uint16_t kNeg136 = 0xC308;      // bf16 -136.0

// (x & 0x000F000F) | kMagic as one v_bitop3 (truth table 0xEA = (a & b) | c);
// written as two operations the compiler emits an AND and an OR with literals
__device__ __forceinline__ uint32_t nib_to_bf16x2(uint32_t x) {
    return __builtin_amdgcn_bitop3_b32(x, 0x000F000Fu, kMagic, 0xEA);
}

__device__ __forceinline__ bf16x8 unpack_codes(uint32_t w) {
    u32x4 r;
    r[0] = nib_to_bf16x2(w);
    r[1] = nib_to_bf16x2(w >> 4);
    r[2] = nib_to_bf16x2(w >> 8);
    r[3] = nib_to_bf16x2(w >> 12);
    return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// Work item `tile` -> (group, first permuted row, row count).  Group g owns
// ceil(n_g / rows_per_tile) consecutive work items.  Every wave computes it.
__device__ __forceinline__ bool find_tile(int tile, int rows_per_tile,
                                          const int32_t *__restrict__ offsets, int G, int &g_out,
                                          int &m0, int &mrows) {
    const int l = lane_id();
    int before = 0;
    for (int g0 = 0; g0 < G; g0 += kWave) {
        const int g = g0 + l;
        int n = 0, lo = 0;
        if (g < G) {
            lo = offsets[g];
            n = offsets[g + 1] - lo;
        }
        const int nt = n > 0 ? (n + rows_per_tile - 1) / rows_per_tile : 0;
        const int incl = wave_incl_scan(nt);
        const int total = __shfl(incl, kWave - 1, kWave);
        if (tile < before + total) {
            const bool mine = g < G && tile >= before + incl - nt && tile < before + incl;
            const uint64_t bal = __ballot(mine);
            const int src = __ffsll((unsigned long long)bal) - 1;
            const int chunk = tile - before - (__shfl(incl, src, kWave) - __shfl(nt, src, kWave));
            g_out = g0 + src;
            const int lo_s = __shfl(lo, src, kWave), n_s = __shfl(n, src, kWave);
            m0 = lo_s + chunk * rows_per_tile;
            mrows = min(rows_per_tile, n_s - chunk * rows_per_tile);
            return true;
        }
        before += total;
    }
    return false;
}

// Same, when every group has at most one work item (T <= rows per tile): the
// work items are the non-empty groups in order, so a ballot and a popcount
// replace the prefix scan.
__device__ __forceinline__ bool find_tile_single(int tile, const int32_t *__restrict__ offsets,
                                                 int G, int &g_out, int &m0, int &mrows) {
    const int l = lane_id();
    int before = 0;
    for (int g0 = 0; g0 < G; g0 += kWave) {
        const int g = g0 + l;
        int n = 0, lo = 0;
        if (g < G) {
            lo = offsets[g];
            n = offsets[g + 1] - lo;
        }
        const uint64_t busy = __ballot(n > 0);
        const int cnt = __popcll(busy);
        if (tile < before + cnt) {
            const int rank = __popcll(busy & ((1ull << l) - 1ull));
            const uint64_t hit = __ballot(n > 0 && rank == tile - before);
            const int src = __ffsll((unsigned long long)hit) - 1;
            g_out = g0 + src;
            m0 = __shfl(lo, src, kWave);
            mrows = __shfl(n, src, kWave);  // the caller bounds it by the tile height
            return true;
        }
        before += cnt;
    }
    return false;
}

// Permuted rows per work item (the MFMA tile has 16; only the first ROWS are
// staged): 1 for single-token decode, else 4 or 8 -- bounded by the
// registers that hold a wave's activation slice while its loads land.
inline int stream_rows_for(int T) { return T <= 1 ? 1 : T <= 4 ? 4 : 8; }

// 16-row weight subtiles per workgroup: 2 while a work item has at most 4
// rows (more, lighter workgroups stream at once), 4 with 8 rows (halves the
// activation re-reads per weight byte).
inline int stream_nsub_for(int T) { return stream_rows_for(T) <= 4 ? 2 : 4; }

// k groups per wave: K/128 is split evenly over at most 4 waves in slices of
// 1, 2, 4 or 8 (0 = unsupported K).
inline int stream_kgw(int KG) {
    for (int kgw = 1; kgw <= 8; kgw *= 2)
        if (KG % kgw == 0 && KG / kgw <= 4) return kgw;
    return 0;
}

// Each wave owns KGW consecutive 128-wide k groups (the host launches
// K/128/KGW waves).  Vector loads of one wave complete in issue order, so a
// wave issues, in this order: its activation slice when every source row
// fits the tile (PRELOAD: before the tile is even known), the scales and
// weights of its first k group, its activation slice otherwise, then the
// rest of its weights; the MFMAs consume the weight stream in issue order
// while later loads are still in flight.  Token indices come through scalar
// loads, which vmcnt does not count.
template <int ACT, int KGW, int ROWS, int NSUB>
__global__ __launch_bounds__(256) void k_w4a16_stream(
    const uint16_t *__restrict__ a, const int32_t *__restrict__ gather, int n_src,
    const u32x4 *__restrict__ wq, const uint16_t *__restrict__ scales,
    const int32_t *__restrict__ offsets, int G, int R, int N, int K, uint16_t *__restrict__ out,
    int NB, bool single) {
    extern __shared__ u32x4 smem[];
    const int nw = blockDim.x >> 6;
    const int wave = threadIdx.x >> 6;
    const int l = lane_id();
    const int m = l & 15, q = l >> 4;
    const int KG = K >> 7, NT = N >> 4;
    const int kg_begin = wave * KGW;

    // activation slice of this wave: [ROWS + 1][KGW*128 + 8] bf16 in LDS; the
    // extra row takes the stores of lanes past the last row, so no store is
    // conditional and no load gets sunk behind one
    constexpr int kSlice = KGW * 128;
    constexpr int kStride = kSlice + 8;
    constexpr int kChunks = kSlice / 8;  // 16-byte chunks per row
    constexpr int kStage = (kChunks * ROWS + kWave - 1) / kWave;
    uint16_t *As = (uint16_t *)smem + (size_t)wave * (ROWS + 1) * kStride;
    u32x4 stage[kStage];

    // (0) PRELOAD: every source row fits the tile -> stage rows 0..n_src-1
    const bool preload = gather != nullptr && n_src <= ROWS;
    if (preload) {
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            const int idx = l + i * kWave;
            const int r = idx / kChunks, c = idx - r * kChunks;
            const int sr = r < n_src ? r : 0;
            stage[i] = *(const u32x4 *)(a + (size_t)sr * K + kg_begin * 128 + 8 * c);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    const int tile = blockIdx.x / NB;
    const int nb = blockIdx.x - tile * NB;
    int g, m0, mrows;
    const bool found = single ? find_tile_single(tile, offsets, G, g, m0, mrows)
                              : find_tile(tile, ROWS, offsets, G, g, m0, mrows);
    if (!found) return;  // uniform over the block
    if (m0 < 0 || m0 >= R) return;                                  // offsets not from moe_permute
    g = __builtin_amdgcn_readfirstlane(g);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    mrows = __builtin_amdgcn_readfirstlane(min(min(mrows, ROWS), R - m0));

    int nrow[NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
        if (ACT == MOE_ACT_SWIGLU) {
            constexpr int half = NSUB / 2;
            const int c = nb * 16 * half + 16 * (s % half);
            nrow[s] = s < half ? c : (N >> 1) + c;
        } else {
            nrow[s] = nb * 16 * NSUB + 16 * s;
        }
    }
    const u32x4 *wg = wq + (size_t)g * NT * KG * kWave;
    const uint16_t *sg = scales + (size_t)g * N * KG;

    // (1) source rows of the tile through scalar loads
    int src[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        src[r] = -1;
        if (r < mrows) {
            if (gather) {
                const int t = gather[m0 + r];
                src[r] = (unsigned)t < (unsigned)n_src ? t : -1;
            } else {
                src[r] = m0 + r;
            }
        }
    }

    // (2) scales of the wave's k range (raw fp16, one vector load per subtile,
    //     converted at use), then the weights of its first k group
    uint16_t sraw[KGW][NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
        const uint16_t *sp = sg + (size_t)(nrow[s] + m) * KG + kg_begin;
        if constexpr (KGW == 8) {
            const u32x4 v = *(const u32x4 *)sp;
#pragma unroll
            for (int j = 0; j < 8; ++j) sraw[j][s] = (uint16_t)(v[j >> 1] >> (16 * (j & 1)));
        } else if constexpr (KGW == 4) {
            const uint2 v = *(const uint2 *)sp;
            sraw[0][s] = (uint16_t)v.x;
            sraw[1][s] = (uint16_t)(v.x >> 16);
            sraw[2][s] = (uint16_t)v.y;
            sraw[3][s] = (uint16_t)(v.y >> 16);
        } else if constexpr (KGW == 2) {
            const uint32_t v = *(const uint32_t *)sp;
            sraw[0][s] = (uint16_t)v;
            sraw[1][s] = (uint16_t)(v >> 16);
        } else {
            sraw[0][s] = *sp;
        }
    }
    u32x4 wv[KGW][NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) wv[0][s] = wg[((size_t)(nrow[s] >> 4) * KG + kg_begin) * kWave + l];
    __builtin_amdgcn_sched_barrier(0);

    // (3) otherwise: the tile's rows x the wave's k slice (unconditional loads,
    //     a divergent load would stall the weight stream; rows past the tile or
    //     with an invalid index are masked at use)
    if (!preload) {
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            const int idx = l + i * kWave;
            const int r = idx / kChunks, c = idx - r * kChunks;
            int sr = src[0] >= 0 ? src[0] : 0;  // unused rows re-read row 0 (an L1 hit)
#pragma unroll
            for (int rr = 1; rr < ROWS; ++rr)
                if (r == rr && src[rr] >= 0) sr = src[rr];
            stage[i] = *(const u32x4 *)(a + (size_t)sr * K + kg_begin * 128 + 8 * c);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // (4) the rest of the wave's weights
#pragma unroll
    for (int j = 1; j < KGW; ++j)
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
            wv[j][s] = wg[((size_t)(nrow[s] >> 4) * KG + kg_begin + j) * kWave + l];
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int i = 0; i < kStage; ++i) {
        const int idx = l + i * kWave;
        const int r = idx / kChunks, c = idx - r * kChunks;
        *(u32x4 *)(As + min(r, ROWS) * kStride + 8 * c) = stage[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // LDS row holding this lane's A row (tile row m): the token itself when
    // preloaded, the tile row otherwise; -1 when the row is absent or invalid
    int arow = -1;
#pragma unroll
    for (int rr = 0; rr < ROWS; ++rr)
        if (m == rr && rr < mrows && src[rr] >= 0) arow = preload ? src[rr] : rr;

    // (5) MFMA over the wave's k range, in load order
    bf16x8 bneg;
#pragma unroll
    for (int i = 0; i < 8; ++i) bneg[i] = __builtin_bit_cast(__bf16, kNeg136);
    f32x4 acc[NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KGW; ++j) {
        u32x4 av[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            av[d] = *(const u32x4 *)(As + max(arow, 0) * kStride + j * 128 + 32 * q + 8 * d);
            if (arow < 0) av[d] = u32x4{0u, 0u, 0u, 0u};
        }
        f32x4 nc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int d = 0; d < 4; ++d) nc = mfma16(__builtin_bit_cast(bf16x8, av[d]), bneg, nc);
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            f32x4 t = nc;
#pragma unroll
            for (int d = 0; d < 4; ++d)
                t = mfma16(__builtin_bit_cast(bf16x8, av[d]), unpack_codes(wv[j][s][d]), t);
            const float sc = half_bits_to_f32(sraw[j][s]);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[s][i] = __builtin_fmaf(sc, t[i], acc[s][i]);
        }
    }

    // (6) add the waves' partial tiles (LDS reused) and write the epilogue
    __syncthreads();
    f32x4 *red = (f32x4 *)smem;  // [nw][NSUB][64]
#pragma unroll
    for (int s = 0; s < NSUB; ++s) red[(wave * NSUB + s) * kWave + l] = acc[s];
    __syncthreads();

    if (ACT == MOE_ACT_SWIGLU) {
        constexpr int half = NSUB / 2;
        const int Nh = N >> 1;
        for (int s = wave; s < half; s += nw) {
            f32x4 gt = red[s * kWave + l], up = red[(s + half) * kWave + l];
            for (int w = 1; w < nw; ++w) {
                gt += red[(w * NSUB + s) * kWave + l];
                up += red[(w * NSUB + s + half) * kWave + l];
            }
            const int n = nrow[s] + m;  // gate row == output column
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int mm = 4 * q + i;
                if (mm < mrows) {
                    const float gv = gt[i];
                    const float h = gv * up[i] * __frcp_rn(1.0f + __expf(-gv));
                    out[(size_t)(m0 + mm) * Nh + n] = f32_to_bf16(h);
                }
            }
        }
    } else {
        for (int s = wave; s < NSUB; s += nw) {
            f32x4 v = red[s * kWave + l];
            for (int w = 1; w < nw; ++w) v += red[(w * NSUB + s) * kWave + l];
            const int n = nrow[s] + m;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int mm = 4 * q + i;
                if (mm < mrows) out[(size_t)(m0 + mm) * N + n] = f32_to_bf16(v[i]);
            }
        }
    }
}

struct StreamArgs {
    const uint16_t *a;
    const int32_t *gather;
    int n_src;
    const u32x4 *wq;
    const uint16_t *scales;
    const int32_t *offsets;
    int G, R, N, K;
    uint16_t *out;
    bool single;  // every group fits one work item
};

template <int ACT, int KGW, int ROWS, int NSUB>
void launch_stream(const StreamArgs &p, hipStream_t st) {
    const int nw = (p.K / 128) / KGW;
    const int NB = p.N / (16 * NSUB);
    const int64_t max_tiles = (int64_t)p.R / ROWS + (p.R < p.G ? p.R : p.G);
    size_t lds = (size_t)nw * (ROWS + 1) * (KGW * 128 + 8) * 2;
    const size_t red = (size_t)nw * NSUB * kWave * 16;
    if (red > lds) lds = red;
    hipLaunchKernelGGL((k_w4a16_stream<ACT, KGW, ROWS, NSUB>), dim3((unsigned)(max_tiles * NB)),
                       dim3(64 * nw), lds, st, p.a, p.gather, p.n_src, p.wq, p.scales, p.offsets,
                       p.G, p.R, p.N, p.K, p.out, NB, p.single);
}

template <int ACT, int ROWS, int NSUB>
void launch_stream_kgw(int KGW, const StreamArgs &p, hipStream_t st) {
    switch (KGW) {
        case 8: launch_stream<ACT, 8, ROWS, NSUB>(p, st); break;
        case 4: launch_stream<ACT, 4, ROWS, NSUB>(p, st); break;
        case 2: launch_stream<ACT, 2, ROWS, NSUB>(p, st); break;
        default: launch_stream<ACT, 1, ROWS, NSUB>(p, st); break;
    }
}

template <int ACT, int NSUB>
void launch_stream_rows(int rows, int KGW, const StreamArgs &p, hipStream_t st) {
    switch (rows) {
        case 1: launch_stream_kgw<ACT, 1, NSUB>(KGW, p, st); break;
        case 4: launch_stream_kgw<ACT, 4, NSUB>(KGW, p, st); break;
        default: launch_stream_kgw<ACT, 8, NSUB>(KGW, p, st); break;
    }
}

template <int ACT>
void launch_stream_all(int nsub, int rows, int KGW, const StreamArgs &p, hipStream_t st) {
    if (nsub == 2)
        launch_stream_rows<ACT, 2>(rows, KGW, p, st);
    else
        launch_stream_rows<ACT, 4>(rows, KGW, p, st);
}


// ---------------------------------------------------------------------------
// LDS-tiled kernel (k_w4a16_tiled), the path for large groups (prefill and
// large batches), where the layer is bound by the matrix cores.  One
// workgroup computes a 128 x 128 tile (permuted rows x weight rows) of one
// group over the whole K, four waves in a 2 x 2 layout of 64 x 64.  Per
// 128-wide k group:
//   * the activation tile (128 gathered rows x 128 k, bf16) is staged in a
//     double-buffered LDS tile while the previous k group is computed;
//   * each wave loads its four 16-row weight subtiles (4 KB of the prepacked
//     stream) and unpacks them once, reusing them for its four 16-row m-tiles;
//   * the -136*sum(A) term is one MFMA chain per m-tile, shared by the four
//     n-tiles, and the fp16 scale is applied per k group in fp32.
// m-tiles past the group's last row are skipped, so a ragged last tile costs
// only its 16-row granularity.  The grid is ordered so that the m-tiles of a
// (group, n-block) are 8 workgroups apart -- workgroups are dealt to the 8
// XCDs in turn -- and therefore read the same weights through one L2.
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
    auto issue = [&](auto stage, int kg, auto tracked) {
        constexpr int ST = decltype(stage)::value;
        u32x4 *A = ST == 0 ? sA0 : ST == 1 ? sA1 : sA2;
        u32x4 *B = ST == 0 ? sB0 : ST == 1 ? sB1 : sB2;
        auto ld = [](const void *g, void *lds) {
            if (decltype(tracked)::value)
                dma16(g, lds);
            else
                dma16_untracked(g, lds);
        };
#pragma unroll
        for (int j = 0; j < 8; ++j) ld(arow_ptr[j] + kg * 128, &A[(32 * wave + 4 * j) * 16]);
        ld(bsrc0 + (size_t)kg * kWave, &B[(2 * wave) * kWave]);
        ld(bsrc1 + (size_t)kg * kWave, &B[(2 * wave + 1) * kWave]);
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
        issue(std::integral_constant<int, (ST + 2) % 3>(), min(kg + 2, KG - 1), std::true_type());

        // A wave whose 64 rows are all past the group's end skips the
        // arithmetic; otherwise the step is straight-line code (rows past
        // the end compute values that are never stored) so that the
        // scheduler can overlap one m-tile's scale FMAs and the next
        // m-tile's LDS reads with the current m-tile's MFMAs.
        if (64 * wm >= mrows) return;
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
inline bool use_tiled(int T, int N, int K) { return T >= 256 && N % kTN == 0 && K <= 4096; }

template <int ACT>
void launch_tiled(const StreamArgs &p, hipStream_t st) {
    const int NB = p.N / kTN;
    const int64_t max_tiles = (int64_t)p.R / kTM + (p.R < p.G ? p.R : p.G);
    const int64_t blocks = (max_tiles * NB + 7) / 8 * 8;  // a whole slice per XCD
    hipLaunchKernelGGL((k_w4a16_tiled<ACT>), dim3((unsigned)blocks), dim3(256), 0, st,
                       p.a, p.gather, p.n_src, p.wq, p.scales, p.offsets, p.G, p.R, p.N, p.K, p.out,
                       NB);
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
    if (N < 64 || N % 64 || K < 128 || K % 128 || N > 65536 || K > 4096 || !stream_kgw(K / 128))
        return MOE_ERR_SHAPE;
    if (a_gather && (n_src < 1 || n_src > MOE_MAX_TOKENS)) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    if (!a || !w_packed || !w_scales || !group_offsets || !out) return MOE_ERR_NULL;
    if (!aligned(a, 16) || !aligned(w_packed, 16) || !aligned(w_scales, 2) ||
        !aligned(group_offsets, 4) || !aligned(out, 16) || (a_gather && !aligned(a_gather, 4)))
        return MOE_ERR_ALIGN;
    const int G = desc->n_routed + desc->n_shared;
    const int64_t R = (int64_t)T * (desc->top_k + desc->n_shared);
    const int rows = stream_rows_for(T);
    const int nsub = stream_nsub_for(T);
    const int64_t max_tiles = R / rows + (R < G ? R : G);
    if (max_tiles * (N / (16 * nsub)) > 0x7FFFFFFF) return MOE_ERR_SHAPE;
    StreamArgs p{a, a_gather, n_src, (const u32x4 *)w_packed, w_scales, group_offsets, G, (int)R,
                 N, K, out, T <= rows};
    const int KGW = stream_kgw(K / 128);
    hipStream_t st = (hipStream_t)stream;
    if (use_tiled(T, N, K)) {
        if (act == MOE_ACT_SWIGLU)
            launch_tiled<MOE_ACT_SWIGLU>(p, st);
        else
            launch_tiled<MOE_ACT_NONE>(p, st);
        return launch_status();
    }
    if (act == MOE_ACT_SWIGLU)
        launch_stream_all<MOE_ACT_SWIGLU>(nsub, rows, KGW, p, st);
    else
        launch_stream_all<MOE_ACT_NONE>(nsub, rows, KGW, p, st);
    return launch_status();
}
