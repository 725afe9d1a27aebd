// moe_gemm.hip -- grouped W4A16 GEMM of the expert projections on gfx950.
//
// Method: weight-only INT4 (one fp16 scale per 128 input elements, symmetric;
// model card "canada-quant/DeepSeek-V4-Flash-W4A16-FP8-MTP", "Component
// precisions"), dequantised in registers and multiplied with bf16
// activations on the matrix cores -- the scheme the Marlin kernel applies on
// Hopper ("Throughputmaxxing: DeepSeek-V4-Flash on Isambard-AI", "A pass through
// the model"), redesigned here for CDNA4.
//
// Weight-stream kernel (k_w4a16_stream; k_mxfp4_stream for FP4 experts), the
// path for small groups, where the layer is bound by HBM weight traffic.  One
// workgroup owns n-blocks of 16*NSUB weight rows (for SwiGLU half gate rows
// and the matching up rows) and at most ROWS permuted rows of one group; its
// waves split K and add their partial tiles through LDS at the end.
//   * B operand (weights): each lane reads 16 bytes of a 1 KB block of the
//     prepacked layout, so a wave load is one contiguous 1 KB stream; the
//     codes go straight from HBM to registers (no LDS).
//   * Unpack: a code u = q+8 placed under the bf16 exponent of 128 gives the
//     exact bf16 value 128+u with one AND-OR per pair of codes.  The MFMA
//     then yields sum A*(q+136); the -136*sum(A) term is one extra MFMA
//     chain per k group with a constant -136 B operand, shared by all
//     subtiles, and is fed in as the accumulator input.
//   * Scales: acc += s[n][kg] * tile after each 128-wide k group (fp32).
//   * A operand (activations): each wave loads the rows x its k slice
//     straight into its own LDS region (XOR-swizzled 16-byte chunks).
// v_mfma_f32_16x16x32_bf16: A = 16 rows x 32 k (lane l: row l%16, k slots
// 8*(l/16)..+8), B = 32 k x 16 cols (lane l: col l%16), D = 16x16 fp32 with
// lane l holding rows 4*(l/16)..+4 of column l%16.  Here rows are permuted
// token rows and columns are weight rows.
#include "moe_gemm_common.h"

namespace moe {
namespace {

// Work item `tile` -> (group, first permuted row, row count).  Group g owns
// ceil(n_g / rows_per_tile) consecutive work items.  Every wave computes it.
__device__ __forceinline__ bool find_tile(int tile, int rows_per_tile,
                                          const int32_t *__restrict__ offsets, int G, int &g_out,
                                          int &m0, int &mrows) {
    int lo[kGroupChunks], n[kGroupChunks];
    load_group_sizes(offsets, G, lo, n);
    int before = 0;
#pragma unroll
    for (int c = 0; c < kGroupChunks; ++c) {
        if (kWave * c >= G) break;
        const int nt = n[c] > 0 ? (n[c] + rows_per_tile - 1) / rows_per_tile : 0;
        const int incl = wave_incl_scan(nt);
        const int total = __shfl(incl, kWave - 1, kWave);
        if (tile < before + total) {
            const bool mine = tile >= before + incl - nt && tile < before + incl;
            const uint64_t bal = __ballot(mine);
            const int src = __ffsll((unsigned long long)bal) - 1;
            const int chunk = tile - before - (__shfl(incl, src, kWave) - __shfl(nt, src, kWave));
            g_out = kWave * c + src;
            const int lo_s = __shfl(lo[c], src, kWave), n_s = __shfl(n[c], src, kWave);
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
    int lo[kGroupChunks], n[kGroupChunks];
    load_group_sizes(offsets, G, lo, n);
    int before = 0;
#pragma unroll
    for (int c = 0; c < kGroupChunks; ++c) {
        if (kWave * c >= G) break;
        const uint64_t busy = __ballot(n[c] > 0);
        const int cnt = __popcll(busy);
        if (tile < before + cnt) {
            const int rank = __popcll(busy & ((1ull << l) - 1ull));
            const uint64_t hit = __ballot(n[c] > 0 && rank == tile - before);
            const int src = __ffsll((unsigned long long)hit) - 1;
            g_out = kWave * c + src;
            m0 = __shfl(lo[c], src, kWave);
            mrows = __shfl(n[c], src, kWave);  // the caller bounds it by the tile height
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

// k groups per wave: slices of 8 whenever that gives at least two waves
// (K/128 = 16: two waves instead of four of 4; the down projection at 64
// tokens 93 -> 87 us), else K/128 split evenly over at most 4 waves in
// slices of 1, 2 or 4 (0 = unsupported K).
inline int stream_kgw(int KG) {
    if (KG % 8 == 0 && KG >= 16 && KG <= 32) return 8;
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
// The activation slice goes from global memory straight into the wave's LDS
// region (16 bytes a lane, 64 chunks per load instruction), so it occupies
// no registers and needs no LDS stores.  Lanes without a row (past the tile,
// or whose token index is invalid) read row 0: a row of A only reaches the
// same row of the product, and those rows are stored as zeros or not at all.
// FMT: kFmtInt4 (fp16 scale per 128 along K, applied per k group, -136
// offset term) or kFmtFp4 (UE8M0 scale per 32 folded into the conversion to
// bf16; the products accumulate directly).
template <int FMT, int ACT, int KGW, int ROWS, int NSUB>
__device__ __forceinline__ void stream_body(
    const uint16_t *__restrict__ a, const int32_t *__restrict__ gather, int n_src,
    const u32x4 *__restrict__ wq, const void *__restrict__ scales,
    const int32_t *__restrict__ offsets, int G, int R, int N, int K, uint16_t *__restrict__ out,
    int NB, int NBW, bool single) {
    extern __shared__ u32x4 smem[];
    const int nw = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = lane_id();
    const int m = l & 15, q = l >> 4;
    const int KG = K >> 7, NT = N >> 4;
    const int kg_begin = wave * KGW;

    // activation slice of this wave: [ROWS][CH] 16-byte chunks in LDS, chunk
    // c of row r at position c ^ lds_swz(r) (conflict-free operand reads)
    constexpr int CH = KGW * 16;
    constexpr int NDMA = (ROWS * CH + kWave - 1) / kWave;
    u32x4 *As = smem + (size_t)wave * ROWS * CH;
    f32x4 *red = (f32x4 *)(smem + (size_t)nw * ROWS * CH);  // [nw - 1][NSUB][64]: waves 1.. partial tiles
    const uint16_t *aslice = a + (size_t)kg_begin * 128;
    // load instruction i fills positions [64i, 64i + 64) of the region, flat
    // over rows; row r is read from source row srow(r) (rows >= nrows skipped)
    auto load_slice = [&](auto srow, int nrows) {
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            if constexpr (CH % kWave == 0) {
                const int r = i * kWave / CH;  // whole instructions per row: a constant
                const int c = (i * kWave) % CH + l;
                if (r < nrows) dma16_untracked(aslice + (size_t)srow(r) * K + 8 * (c ^ lds_swz(r)), As + i * kWave);
            } else {
                const int f = i * kWave + l, r = f / CH, c = f - r * CH;
                if (r < nrows) {
                    int sr = srow(0);
#pragma unroll
                    for (int rr = 1; rr < ROWS; ++rr)
                        if (r == rr) sr = srow(rr);
                    dma16_untracked(aslice + (size_t)sr * K + 8 * (c ^ lds_swz(r)), As + i * kWave);
                }
            }
        }
    };

    // (0) PRELOAD: every source row fits the tile -> rows 0..n_src-1
    const bool preload = gather != nullptr && n_src <= ROWS;
    if (preload) load_slice([](int r) { return r; }, n_src);
    __builtin_amdgcn_sched_barrier(0);

    // block -> (tile, n-block set); the block takes n-blocks nbb, nbb + NBB,
    // ... (NBW of them) of one tile, finding the tile and loading its
    // activation slice once
    const int NBB = NB / NBW;
    const int tile = blockIdx.x / NBB;
    const int nbb = blockIdx.x - tile * NBB;
    int g, m0, mrows;
    const bool found = single ? find_tile_single(tile, offsets, G, g, m0, mrows)
                              : find_tile(tile, ROWS, offsets, G, g, m0, mrows);
    // uniform over the block; no load into LDS may outlive it
    if (!found || m0 < 0 || m0 >= R) {  // (m0 outside: offsets not from moe_permute)
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }
    g = __builtin_amdgcn_readfirstlane(g);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    mrows = __builtin_amdgcn_readfirstlane(min(min(mrows, ROWS), R - m0));
    const u32x4 *wg = wq + (size_t)g * NT * KG * kWave;
    const uint16_t *sg = (const uint16_t *)scales + (size_t)g * N * KG;       // INT4: fp16 [N][KG]
    const uint8_t *sg8 = (const uint8_t *)scales + (size_t)g * N * (K >> 5);  // FP4: UE8M0 [N][K/32]

    // (1) source rows of the tile through scalar loads; bit r of `valid`:
    //     row r exists and has a valid token index
    int src[ROWS];
    uint32_t valid = 0;
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
        if (src[r] >= 0) valid |= 1u << r;
    }
    // LDS row holding this lane's A row (tile row m): the token itself when
    // preloaded, the tile row otherwise; row 0 when the row is absent
    int arow = 0;
#pragma unroll
    for (int rr = 0; rr < ROWS; ++rr)
        if (m == rr && src[rr] >= 0) arow = preload ? src[rr] : rr;
    const u32x4 *Arow = As + arow * CH;
    const int asw = lds_swz(arow);

    for (int u = 0; u < NBW; ++u) {
        const int nb = nbb + u * NBB;
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

        // (2) scales of the wave's k range (raw fp16, one vector load per
        //     subtile, converted at use), then the weights of its first k group
        // INT4: fp16 scale of (row, k group); FP4: the scale bytes of the row's
        // 32-wide blocks over the wave's k range, dword j holding k group j
        // (this lane's block q is byte q)
        uint16_t sraw[KGW][NSUB];
        uint32_t sblk[KGW][NSUB];
        if constexpr (FMT == kFmtInt4) {
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
        } else {
#pragma unroll
            for (int s = 0; s < NSUB; ++s) {
                const uint8_t *sp = sg8 + (size_t)(nrow[s] + m) * (K >> 5) + 4 * kg_begin;
                if constexpr (KGW >= 4) {
#pragma unroll
                    for (int j0 = 0; j0 < KGW; j0 += 4) {
                        const u32x4 v = *(const u32x4 *)(sp + 4 * j0);
#pragma unroll
                        for (int j = 0; j < 4; ++j) sblk[j0 + j][s] = v[j];
                    }
                } else if constexpr (KGW == 2) {
                    const uint2 v = *(const uint2 *)sp;
                    sblk[0][s] = v.x;
                    sblk[1][s] = v.y;
                } else {
                    sblk[0][s] = *(const uint32_t *)sp;
                }
            }
        }
        // weight subtile s of this wave's k range: a wave-uniform base, lane
        // l's 16 bytes of each 1 KB block at +16*l
        const u32x4 *wb[NSUB];
#pragma unroll
        for (int s = 0; s < NSUB; ++s) wb[s] = wg + ((size_t)(nrow[s] >> 4) * KG + kg_begin) * kWave;
        u32x4 wv[KGW][NSUB];
#pragma unroll
        for (int s = 0; s < NSUB; ++s) wv[0][s] = wb[s][l];
        __builtin_amdgcn_sched_barrier(0);

        // (3) first n-block, no preload: the tile's rows x the wave's k slice
        //     (a row without a valid token reads token 0; it is never used)
        if (u == 0 && !preload) load_slice([&](int r) { return max(src[r], 0); }, mrows);
        __builtin_amdgcn_sched_barrier(0);

        // (4) the rest of the wave's weights
#pragma unroll
        for (int j = 1; j < KGW; ++j)
#pragma unroll
            for (int s = 0; s < NSUB; ++s) wv[j][s] = wb[s][j * kWave + l];
        // the slice has landed once at most the later weight loads are in flight
        if (u == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm((KGW - 1) * NSUB));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);

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
            for (int d = 0; d < 4; ++d) av[d] = Arow[16 * j + ((4 * q + d) ^ asw)];
            if constexpr (FMT == kFmtFp4) {
#pragma unroll
                for (int s = 0; s < NSUB; ++s) {
                    const float e = ue8m0_to_f32((sblk[j][s] >> (8 * q)) & 0xFFu);
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        acc[s] = mfma16(__builtin_bit_cast(bf16x8, av[d]), fp4x8_to_bf16(wv[j][s][d], e), acc[s]);
                }
                continue;
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

        // (6) waves 1.. hand their partial tiles to wave 0 through LDS, which
        //     adds them to its own and writes the epilogue; the barrier before
        //     the handover keeps it from overwriting what wave 0 still reads
        __syncthreads();
        if (wave > 0) {
#pragma unroll
            for (int s = 0; s < NSUB; ++s) red[((wave - 1) * NSUB + s) * kWave + l] = acc[s];
        }
        __syncthreads();
        if (wave == 0) {
            for (int w = 1; w < nw; ++w)
#pragma unroll
                for (int s = 0; s < NSUB; ++s) acc[s] += red[((w - 1) * NSUB + s) * kWave + l];
            if (ACT == MOE_ACT_SWIGLU) {
                constexpr int half = NSUB / 2;
                const int Nh = N >> 1;
#pragma unroll
                for (int s = 0; s < half; ++s) {
                    const int n = nrow[s] + m;  // gate row == output column
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int mm = 4 * q + i;
                        if (mm < mrows) {
                            const float gv = acc[s][i];
                            const float h = silu_mul(gv, acc[s + half][i]);
                            out[(size_t)(m0 + mm) * Nh + n] = (valid >> mm) & 1u ? f32_to_bf16(h) : (uint16_t)0;
                        }
                    }
                }
            } else {
#pragma unroll
                for (int s = 0; s < NSUB; ++s) {
                    const int n = nrow[s] + m;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int mm = 4 * q + i;
                        if (mm < mrows)
                            out[(size_t)(m0 + mm) * N + n] = (valid >> mm) & 1u ? f32_to_bf16(acc[s][i]) : (uint16_t)0;
                    }
                }
            }
        }
    }
}


// n-blocks per workgroup: the grid covers the worst case (every group a
// partial tile), and at 64 tokens that is three times the tiles a routing
// makes; a workgroup launched only to find no work costs about as much as a
// short one.  A workgroup takes n-blocks nbb, nbb + NB/nbw, ... of its tile
// (the tile found and its activations loaded once).  Measured on whole
// layers (iid routing): 2 while groups average under half a row (the launch
// is small anyway; 8 and 16 tokens 134 -> 124, 220 -> 192 us against one),
// 4 under one row (32 tokens 319 -> 240 us), 8 from there (64 tokens
// 163 -> 158 us for the gate/up against 4; 16 was no better at 128 tokens).
inline int stream_nbw(int64_t R, int G, int NB) {
    const int want = 2 * R < G ? 2 : R < G ? 4 : 8;
    for (int n = want; n > 1; n >>= 1)
        if (NB % n == 0) return n;
    return 1;
}

#define MOE_STREAM_ARGS                                                                           \
    const uint16_t *__restrict__ a, const int32_t *__restrict__ gather, int n_src,                \
        const u32x4 *__restrict__ wq, const void *__restrict__ scales,                            \
        const int32_t *__restrict__ offsets, int G, int R, int N, int K, uint16_t *__restrict__ out, \
        int NB, int NBW, bool single
#define MOE_STREAM_PASS a, gather, n_src, wq, scales, offsets, G, R, N, K, out, NB, NBW, single

template <int ACT, int KGW, int ROWS, int NSUB>
__global__ __launch_bounds__(256) void k_w4a16_stream(MOE_STREAM_ARGS) {
    stream_body<kFmtInt4, ACT, KGW, ROWS, NSUB>(MOE_STREAM_PASS);
}

template <int ACT, int KGW, int ROWS, int NSUB>
__global__ __launch_bounds__(256) void k_mxfp4_stream(MOE_STREAM_ARGS) {
    stream_body<kFmtFp4, ACT, KGW, ROWS, NSUB>(MOE_STREAM_PASS);
}

template <int ACT, int KGW, int ROWS, int NSUB>
void launch_stream(const GemmArgs &p, hipStream_t st) {
    const int nw = (p.K / 128) / KGW;
    const int NB = p.N / (16 * NSUB);
    const int64_t max_tiles = (int64_t)p.R / ROWS + (p.R < p.G ? p.R : p.G);
    const size_t lds = (size_t)nw * ROWS * KGW * 128 * 2 + (size_t)(nw - 1) * NSUB * kWave * 16;
    const int nbw = stream_nbw(p.R, p.G, NB);
    auto kern = p.fp4 ? k_mxfp4_stream<ACT, KGW, ROWS, NSUB> : k_w4a16_stream<ACT, KGW, ROWS, NSUB>;
    hipLaunchKernelGGL(kern, dim3((unsigned)(max_tiles * (NB / nbw))), dim3(64 * nw), lds, st, p.a, p.gather,
                       p.n_src, p.wq, p.scales, p.offsets, p.G, p.R, p.N, p.K, p.out, NB, nbw, p.single);
}

template <int ACT, int ROWS, int NSUB>
void launch_stream_kgw(int KGW, const GemmArgs &p, hipStream_t st) {
    switch (KGW) {
        case 8: launch_stream<ACT, 8, ROWS, NSUB>(p, st); break;
        case 4: launch_stream<ACT, 4, ROWS, NSUB>(p, st); break;
        case 2: launch_stream<ACT, 2, ROWS, NSUB>(p, st); break;
        default: launch_stream<ACT, 1, ROWS, NSUB>(p, st); break;
    }
}

template <int ACT, int NSUB>
void launch_stream_rows(int rows, int KGW, const GemmArgs &p, hipStream_t st) {
    switch (rows) {
        case 1: launch_stream_kgw<ACT, 1, NSUB>(KGW, p, st); break;
        case 4: launch_stream_kgw<ACT, 4, NSUB>(KGW, p, st); break;
        default: launch_stream_kgw<ACT, 8, NSUB>(KGW, p, st); break;
    }
}

template <int ACT>
void launch_stream_all(int nsub, int rows, int KGW, const GemmArgs &p, hipStream_t st) {
    if (nsub == 2)
        launch_stream_rows<ACT, 2>(rows, KGW, p, st);
    else
        launch_stream_rows<ACT, 4>(rows, KGW, p, st);
}


}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_w4a16_grouped_gemm(const moe_layer_desc *desc, int32_t T,
                                             const uint16_t *a, const int32_t *a_gather,
                                             int32_t n_src, const float *a_sums, int32_t N,
                                             int32_t K, const uint8_t *w_packed,
                                             const uint16_t *w_scales, const int32_t *group_offsets,
                                             int32_t act, uint16_t *out, void *stream) {
    MOE_TRY(check_desc(desc));
    MOE_TRY(check_tokens(T));
    if (act != MOE_ACT_NONE && act != MOE_ACT_SWIGLU) return MOE_ERR_UNSUPPORTED;
    if (N < 64 || N % 64 || K < 128 || K % 128 || N > 65536 || K > 4096 || !stream_kgw(K / 128))
        return MOE_ERR_SHAPE;
    if (a_gather && (n_src < 1 || n_src > MOE_MAX_TOKENS)) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    if (!a || !w_packed || !w_scales || !group_offsets || !out) return MOE_ERR_NULL;
    if (!aligned(a, 16) || !aligned(w_packed, 16) || !aligned(w_scales, 2) ||
        !aligned(group_offsets, 4) || !aligned(out, 16) || (a_gather && !aligned(a_gather, 4)) ||
        (a_sums && !aligned(a_sums, 4)))
        return MOE_ERR_ALIGN;
    const int G = desc->n_routed + desc->n_shared;
    const int64_t R = (int64_t)T * (desc->top_k + desc->n_shared);
    const int rows = stream_rows_for(T);
    const int nsub = stream_nsub_for(T);
    const int64_t max_tiles = R / rows + (R < G ? R : G);
    if (max_tiles * (N / (16 * nsub)) > 0x7FFFFFFF) return MOE_ERR_SHAPE;
    GemmArgs p{a, a_gather, n_src, (const u32x4 *)w_packed, w_scales, group_offsets, G, (int)R,
                 N, K, out, T <= rows, T >= MOE_TILED_MIN_TOKENS ? a_sums : nullptr};
    const int KGW = stream_kgw(K / 128);
    hipStream_t st = (hipStream_t)stream;
    if (use_tiled(T, N, K)) {
        launch_tiled(act, p, st);
        return launch_status();
    }
    if (act == MOE_ACT_SWIGLU)
        launch_stream_all<MOE_ACT_SWIGLU>(nsub, rows, KGW, p, st);
    else
        launch_stream_all<MOE_ACT_NONE>(nsub, rows, KGW, p, st);
    return launch_status();
}

extern "C" moe_status moe_mxfp4_grouped_gemm(const moe_layer_desc *desc, int32_t T,
                                             const uint16_t *a, const int32_t *a_gather,
                                             int32_t n_src, int32_t N, int32_t K,
                                             const uint8_t *w_packed, const uint8_t *w_scales,
                                             const int32_t *group_offsets, int32_t act,
                                             uint16_t *out, void *stream) {
    MOE_TRY(check_desc(desc));
    MOE_TRY(check_tokens(T));
    if (act != MOE_ACT_NONE && act != MOE_ACT_SWIGLU) return MOE_ERR_UNSUPPORTED;
    if (N < 128 || N % 128 || K < 128 || K % 128 || N > 65536 || K > 4096) return MOE_ERR_SHAPE;
    if (a_gather && (n_src < 1 || n_src > MOE_MAX_TOKENS)) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    if (!a || !w_packed || !w_scales || !group_offsets || !out) return MOE_ERR_NULL;
    if (!aligned(a, 16) || !aligned(w_packed, 16) || !aligned(w_scales, 16) || !aligned(group_offsets, 4) ||
        !aligned(out, 16) || (a_gather && !aligned(a_gather, 4)))
        return MOE_ERR_ALIGN;
    const int G = desc->n_routed + desc->n_shared;
    const int64_t R = (int64_t)T * (desc->top_k + desc->n_shared);
    const int KGW = stream_kgw(K / 128);
    hipStream_t st = (hipStream_t)stream;
    if (use_tiled(T, N, K) || !KGW) {
        const int64_t max_tiles = R / 64 + (R < G ? R : G);
        if (max_tiles * (N / 128) > 0x7FFFFFFF) return MOE_ERR_SHAPE;
        GemmArgs p{a, a_gather, n_src, (const u32x4 *)w_packed, w_scales, group_offsets, G, (int)R,
                   N, K, out, false, nullptr, true};
        launch_tiled(act, p, st, true);
        return launch_status();
    }
    const int rows = stream_rows_for(T);
    const int nsub = stream_nsub_for(T);
    const int64_t max_tiles = R / rows + (R < G ? R : G);
    if (max_tiles * (N / (16 * nsub)) > 0x7FFFFFFF) return MOE_ERR_SHAPE;
    GemmArgs p{a, a_gather, n_src, (const u32x4 *)w_packed, w_scales, group_offsets, G, (int)R,
               N, K, out, T <= rows, nullptr, true};
    if (act == MOE_ACT_SWIGLU)
        launch_stream_all<MOE_ACT_SWIGLU>(nsub, rows, KGW, p, st);
    else
        launch_stream_all<MOE_ACT_NONE>(nsub, rows, KGW, p, st);
    return launch_status();
}

// ---------------------------------------------------------------------------
// Row sums over 128-wide k groups (the a_sums input of the GEMM).  One wave
// per row; each lane adds its eight consecutive elements in order, then the
// sixteen lanes of a group combine by pairwise halving (xor 8, 4, 2, 1).
namespace moe {
namespace {
__global__ __launch_bounds__(256) void k_row_sums(const uint16_t *__restrict__ a, int rows, int K,
                                                  float *__restrict__ sums) {
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    const int l = lane_id();
    const uint16_t *row = a + (size_t)r * K;
    const int KG = K >> 7;
    for (int c = 0; c < K; c += 8 * kWave) {
        float s = 0.0f;
        const bool in = c + 8 * l < K;  // K is a multiple of 128: whole groups in or out
        if (in) {
            const u32x4 v = *(const u32x4 *)(row + c + 8 * l);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s += bf16lo_to_f32(v[i]);
                s += bf16hi_to_f32(v[i]);
            }
        }
#pragma unroll
        for (int d = 8; d >= 1; d >>= 1) s += __shfl_xor(s, d, kWave);
        if (in && (l & 15) == 0) sums[(size_t)r * KG + (c >> 7) + (l >> 4)] = s;
    }
}
}  // namespace
}  // namespace moe

extern "C" moe_status moe_row_sums(int32_t rows, int32_t K, const uint16_t *a, float *sums,
                                   void *stream) {
    if (rows < 0 || (int64_t)rows > (int64_t)MOE_MAX_TOKENS * 9 || K < 128 || K % 128 || K > 65536)
        return MOE_ERR_SHAPE;
    if (rows == 0) return MOE_OK;
    if (!a || !sums) return MOE_ERR_NULL;
    if (!aligned(a, 16) || !aligned(sums, 4)) return MOE_ERR_ALIGN;
    hipLaunchKernelGGL(k_row_sums, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, (hipStream_t)stream,
                       a, rows, K, sums);
    return launch_status();
}
