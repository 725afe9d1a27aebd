// moe_gemm_common.h -- what the two grouped W4A16 GEMM kernels share: the
// INT4 unpack, the MFMA wrapper, the launch arguments, and the entry to the
// tiled kernel (moe_gemm_tiled.hip, compiled with its own scheduling flags).
#pragma once

#include "moe_common.h"

namespace moe {

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

// FMT: kFmtInt4 (INT4 codes as q+8, one fp16 scale per 128 along K, applied
// to each k group's partial sums) or kFmtFp4 (E2M1 codes in natural order,
// one UE8M0 scale per 32 along K, folded into the hardware conversion to
// bf16: the products accumulate with no offset term and no per-group
// scaling).
constexpr int kFmtInt4 = 0, kFmtFp4 = 1;

// eight E2M1 codes (element j in bits [4j, 4j+4)) times the power of two s,
// as bf16 -- exact: two significant bits times a power of two
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t w, float s) {
    const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
    const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
    const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
    const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
    bf16x8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// UE8M0 byte E -> 2^(E-127) as fp32 (E = 0: the subnormal 2^-127)
__device__ __forceinline__ float ue8m0_to_f32(uint32_t E) {
    return __uint_as_float(E == 0u ? 0x00400000u : E << 23);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// 16 bytes per lane straight from global memory into LDS: lane l's bytes land
// at lds + 16*l (the LDS address is wave-uniform); counted by vmcnt.
__device__ __forceinline__ void dma16(const void *g, void *lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void_t *)lds, 16, 0, 0);
}
// The same load written as inline assembly, which the compiler's wait-count
// pass does not track.  Tracked, they make the pass wait for every load into LDS before the
// first LDS read that follows them, however far ahead they were issued; the
// kernels order their completion with explicit waits instead.
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

// x rounded to e4m3 at the block scale 2^(E-127) and back: the value the
// quantised activation stands for (e4m3 has four significant bits, so the
// result is exact in bf16).  The conversion is the one the quantising
// kernel uses (round to nearest even, saturating at 448).
__device__ __forceinline__ float fp8_roundtrip(float x, int E) {
    const float inv = __uint_as_float((uint32_t)(254 - E) << 23);  // 2^-(E-127): exact
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(x * inv, 0.0f, 0, false);
    return __builtin_amdgcn_cvt_f32_fp8(w, 0) * ue8m0_to_f32((uint32_t)E);
}

// SwiGLU of one output column: silu(g) * u = g * u / (1 + e^-g), with the
// hardware exponential and reciprocal (each within an ulp or two of fp32; the
// activation is not bit-specified, the oracle takes fp64, and h is then
// rounded to bf16).  A large negative g gives 1 + e^-g = inf and h = 0.
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// s_waitcnt immediate for "at most n vector-memory operations outstanding"
// (vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// Where the 16-byte chunk c of activation row r sits in LDS: chunk c ^ lds_swz(r).
// A matrix-core operand read takes, for each of its four k slices, rows
// 16i..16i+15 and chunks 4q+d (q = lane/16): 64 lanes over 16 rows.  gfx950
// serves a 16-byte-per-lane LDS read 16 lanes per cycle from 64 four-byte
// banks (256 bytes), the lanes grouped as {0-3, 12-15, 20-23, 24-27},
// {4-11, 16-19, 28-31} and the same plus 32 (measured: these groups explain
// the bank-conflict counter over five access patterns).  With a plain
// "c ^ (r & 15)", lanes 0-3 (rows 0-3, q = 0) and 20-23 (rows 4-7, q = 1)
// land on the same banks, doubling every read; flipping bit 3 of the swizzle
// by bit 2 of the row puts each group on 16 distinct chunks.
__device__ __forceinline__ int lds_swz(int r) {
    const int x = r & 15;
    return x ^ ((x & 4) << 1);
}

// A layer has at most 257 groups (256 routed experts and one shared, checked
// on the host): five chunks of 64.  Lane l holds the first row and the row
// count of groups l, 64+l, ...; every load is issued before any is used, so
// the table costs one memory round trip (a loop that loads a chunk, scans it
// and moves on pays one round trip per chunk, which dominated the life of a
// workgroup that finds no work).
constexpr int kGroupChunks = 5;
static_assert(256 + 1 <= kWave * kGroupChunks, "check_desc admits at most 256 routed experts and one shared");
// (offsets null: one group of rows [0, R), a dense GEMM.)
__device__ __forceinline__ void load_group_sizes(const int32_t *__restrict__ offsets, int G,
                                                 int (&lo)[kGroupChunks], int (&n)[kGroupChunks], int R = 0) {
    const int l = lane_id();
    if (!offsets) {
#pragma unroll
        for (int c = 0; c < kGroupChunks; ++c) {
            lo[c] = 0;
            n[c] = kWave * c + l == 0 ? R : 0;
        }
        return;
    }
    // every entry is loaded (in bounds: offsets has G + 1) before any is
    // used, the lanes past G selected out afterwards: a load under a lane
    // condition, or a use between the loads, would put a wait between them
    int a[kGroupChunks], b[kGroupChunks];
#pragma unroll
    for (int c = 0; c < kGroupChunks; ++c) {
        const int gi = min(kWave * c + l, G);
        a[c] = offsets[gi];
        b[c] = offsets[min(gi + 1, G)];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < kGroupChunks; ++c) {
        const bool in = kWave * c + l < G;
        lo[c] = in ? a[c] : 0;
        n[c] = in ? b[c] - a[c] : 0;
    }
}

// The work list of the LDS-tiled kernels (TM permuted rows x one n-block of
// weight rows per item) and the XCD-aware order in which blocks take it.
__device__ __forceinline__ bool find_tile_item(int b, int NB, int TM, const int32_t *__restrict__ offsets,
                                                int G, int &g_out, int &m0, int &mrows, int &nb, int R = 0) {
    // The work list: groups in order; a group's m-tiles in chunks of up to
    // four; inside a chunk n-block-major, so 32 consecutive items cover 8
    // n-blocks x 4 m-tiles.  Blocks are dealt to the eight XCDs in turn
    // (block b runs on XCD b % 8) and XCD x takes the contiguous slice
    // [x*per, (x+1)*per) of the list, so the blocks resident on one XCD at a
    // time share activation tiles and weight slices in that XCD's L2.
    int lo[kGroupChunks], n[kGroupChunks], mt[kGroupChunks], items[kGroupChunks];
    load_group_sizes(offsets, G, lo, n, R);
    int total = 0;
#pragma unroll
    for (int c = 0; c < kGroupChunks; ++c) {
        mt[c] = n[c] > 0 ? (n[c] + TM - 1) / TM : 0;
        items[c] = mt[c] * NB;
        total += __shfl(wave_incl_scan(items[c]), kWave - 1, kWave);
    }
    const int per = (total + 7) >> 3;
    const int x = b & 7, j = b >> 3;
    const int item = x * per + j;
    if (j >= per || item >= total) return false;
    int before = 0;
#pragma unroll
    for (int c = 0; c < kGroupChunks; ++c) {
        const int incl = wave_incl_scan(items[c]);
        const int tot = __shfl(incl, kWave - 1, kWave);
        if (item < before + tot) {
            const bool mine = item >= before + incl - items[c] && item < before + incl;
            const int src = __ffsll((unsigned long long)__ballot(mine)) - 1;
            const int local = item - before - (__shfl(incl, src, kWave) - __shfl(items[c], src, kWave));
            const int mt_s = __shfl(mt[c], src, kWave);
            const int ch = local / (4 * NB), rem = local - ch * 4 * NB;
            const int mc = min(4, mt_s - 4 * ch);
            const int nbi = rem / mc;
            const int mi = 4 * ch + rem - nbi * mc;
            g_out = kWave * c + src;
            m0 = __shfl(lo[c], src, kWave) + mi * TM;
            mrows = min(TM, __shfl(n[c], src, kWave) - mi * TM);
            nb = nbi;
            return true;
        }
        before += tot;
    }
    return false;
}

// The workgroup's work item: wave 0 searches the work list and hands the item
// to the other waves through LDS (the search is a few hundred vector
// instructions, which the other waves' SIMDs spend on other workgroups
// instead).  False, for the whole workgroup, when there is no item; mrows is
// clamped to the rows that exist.  Contains a workgroup barrier.
struct TileItem {
    int g, m0, mrows, nb;
};
__device__ __forceinline__ bool workgroup_tile_item(int NB, int TM, const int32_t *__restrict__ offsets, int G,
                                                    int R, TileItem &it) {
    __shared__ int sitem[4];
    if ((threadIdx.x >> 6) == 0) {
        int g = 0, m0 = 0, mrows = 0, nb = 0;
        const bool ok = find_tile_item(blockIdx.x, NB, TM, offsets, G, g, m0, mrows, nb, R) && m0 >= 0 && m0 < R;
        if (lane_id() == 0) {
            sitem[0] = ok ? g : -1;
            sitem[1] = m0;
            sitem[2] = mrows;
            sitem[3] = nb;
        }
    }
    __syncthreads();
    it.g = __builtin_amdgcn_readfirstlane(sitem[0]);
    if (it.g < 0) return false;
    it.m0 = __builtin_amdgcn_readfirstlane(sitem[1]);
    it.nb = __builtin_amdgcn_readfirstlane(sitem[3]);
    it.mrows = __builtin_amdgcn_readfirstlane(min(sitem[2], R - it.m0));
    return true;
}

struct GemmArgs {
    const uint16_t *a;
    const int32_t *gather;
    int n_src;
    const u32x4 *wq;
    const void *scales;  // fp16 [G][N][K/128] (INT4) or UE8M0 bytes [G][N][K/32] (FP4)
    const int32_t *offsets;
    int G, R, N, K;
    uint16_t *out;
    bool single;        // every group fits one work item
    const float *sums;  // row sums of a over 128-wide k groups, or null
    bool fp4 = false;   // FP4 weights and scales (else INT4)
};

// The tiled kernel takes groups with many rows: T >= MOE_TILED_MIN_TOKENS, N a
// multiple of its 128-row n-block, K at most 4096 (its scale table in LDS).
bool use_tiled(int T, int N, int K);  // from MOE_TILED_MIN_TOKENS tokens, ...
void launch_tiled(int act, const GemmArgs &p, hipStream_t st, bool fp4 = false);

// FP4 weights on 128 x 512 tiles (moe_gemm_fp4wide.hip): the tiled path's
// kernel for FP4 when N is a multiple of 512, K of 256 (up to 4096) and the
// scales 4-byte aligned.
bool use_fp4_wide(const GemmArgs &p);
void launch_fp4_wide(int act, const GemmArgs &p, hipStream_t st);

}  // namespace moe
