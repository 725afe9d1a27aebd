// moe_decode.hip -- the whole MoE layer for one token in one launch (the
// bs = 1 decode step) on gfx950.
//
// The layer routes the token to k of E experts (sigmoid score plus an FP32
// gate bias; "DeepSeek V4 Flash serving hardware", 01, "Sparse
// architecture"; model card "canada-quant/DeepSeek-V4-Flash-W4A16-FP8-MTP",
// "Component precisions"), runs each chosen expert and the shared expert as
// a SwiGLU MLP with W4A16 weights, and sums the expert outputs with the
// routing weights.  At one token the step is a stream of ~93 MB of INT4
// weights, so HBM must stay busy from the first microsecond to the last.
// As separate launches (route+permute, gate/up, down+combine) each waits for
// the one before and starts with a memory round trip; here one workgroup per
// CU runs the whole step, and what one workgroup needs from the others comes
// through a caller-provided workspace:
//   phase 0 (needs nothing): waves 0..3 compute router logits and publish
//     each expert's score tagged with the call's epoch; x goes to LDS; the
//     first 2*I/16 workgroups stream half a tile of the shared expert's
//     gate/up rows each (8 of its 16 h columns, over all of K).
//   phase 1: wave 0 polls the E tagged scores until all carry this call's
//     epoch and selects the top k experts itself with the selection code of
//     moe_route (a bit-identical choice).  Meanwhile the other waves compute
//     the shared tile.  The routing weights, the permuted rows and (in
//     workgroup 0) the routing outputs follow in phase 2, once wave 0's own
//     loads are issued: only the experts gate the stream.
//   phase 2: waves 0..11 stream the routed gate/up tiles (16 h columns x all
//     of K each, four waves per tile splitting K; 3 tiles per workgroup at
//     full size) and write h; waves 12..15 load the down rows and scales of
//     the workgroup's 16 output columns, for every slot, straight into LDS.
//     Every h tile (routed and shared) is also written to the workspace as
//     64-bit words (two bf16 values and the call's epoch tag).
//   phase 3: once the workgroup's down rows are in LDS, each wave polls the
//     tagged h words of its (slot, k group) pairs until all carry this
//     call's tag, then computes the down projection of the workgroup's 16
//     output columns over them, weighted by the routing weights; the waves'
//     sums are added in order: out.
// Data that crosses workgroups (scores, h) moves with device-coherent stores
// and loads of 64-bit words that carry the call's epoch, so a reader needs
// no separate flag, nothing has to be reset between calls, and no atomic
// read-modify-write is used.  Each score is written to 16 copies, and one
// workgroup in 16 polls each copy.  Every workgroup raises a flag once it
// has read the epoch; workgroup 0 advances the epoch at its end, once every
// flag is up.  Every wait is bounded (100 ms of the real-time clock): a wait
// that runs out raises an error word in the workspace and the kernel still
// runs to its end with in-bounds accesses.
//
// The same kernel takes FP4 experts (E2M1 codes, one UE8M0 scale per 32
// along K; k_mxfp4_decode_token): every weight is converted to bf16 with
// its block scale folded in, so the offset terms and per-group scaling of
// the INT4 codes fall away; the data movement is the same.
//
// A wave's vector loads complete in issue order, and any wait for one of
// them (or an LDS fence while a load into LDS is pending) waits for all
// issued before it.  So the waves that load into LDS issue nothing else in
// phase 2 and pass its barrier without a fence; the gate/up waves issue no
// load into LDS, and their waits for stored h tiles wait only for their own
// (already consumed) weight loads.
#include "moe_gemm_common.h"
#include "moe_route_common.h"

namespace moe {
namespace {

constexpr int kWaves = 16;
constexpr int kMaxTiles = 3;               // routed gate/up tiles per workgroup, 4 waves each
constexpr int kDmaWave0 = 4 * kMaxTiles;   // waves kDmaWave0.. load the down rows into LDS
constexpr int kDmaWaves = kWaves - kDmaWave0;
constexpr int kMaxPairs = 112;  // (slot, down k group) weight blocks held in LDS
constexpr int kPairsPerWave = (kMaxPairs + kWaves - 1) / kWaves;
constexpr int kDmaPerWave = kMaxPairs / kDmaWaves;
static_assert(kDmaPerWave * kDmaWaves == kMaxPairs, "down rows split evenly");
constexpr int kShDmaPerWave = 32 / kDmaWaves;  // the shared expert's pairs: I/128 <= 32
// down scales per slot, in dwords per I/128: 16 rows x one fp16 (INT4) or
// 16 rows x four UE8M0 bytes (FP4); at most kMaxPairs (slot, k group)
// blocks, loaded 64 dwords per instruction
template <int FMT>
constexpr int scale_dwords_per_kg() { return FMT == kFmtInt4 ? 8 : 16; }
template <int FMT>
constexpr int scale_dwords() { return scale_dwords_per_kg<FMT>() * kMaxPairs; }
template <int FMT>
constexpr int scale_dma_per_wave() { return (scale_dwords<FMT>() / 64 + kDmaWaves - 1) / kDmaWaves; }
constexpr uint64_t kWaitTicks = 10000000;  // 100 ms of the 100 MHz real-time counter

// workspace words (MOE_DECODE_WORKSPACE_BYTES in the ABI header).  Each
// score is written to kReplicas copies 4 KB apart, and workgroup b reads
// copy b % kReplicas: no word has more than P/kReplicas readers polling it.
constexpr int kReplicas = 16;
constexpr int kWsErr = 3, kWsEpoch = 4;
constexpr int kWsScores = 1024;                        // [16][512] 64-bit (score, epoch tag)
constexpr int kWsDone = kWsScores + kReplicas * 1024;  // [1024] epoch tag per workgroup
constexpr int kWsHtag = kWsDone + 1024;                // [slot][I/2] 64-bit (bf16 pair, epoch tag)
constexpr int kMaxGrid = 256;                          // workgroups with a score / done slot
static_assert((kWsHtag + 2 * kMaxPairs * 64) * 4 == MOE_DECODE_WORKSPACE_BYTES, "workspace layout");
constexpr int kShWaves = 4 * kMaxTiles - 1;  // waves 1..kShWaves compute the shared tile

// LDS region reused between phases: phases 0..2 hold x (8 KB) and the
// partial tiles of the waves; phase 3 the h slices of every wave's pairs
constexpr int kRedT = 2048;                          // float offset of [kMaxTiles][2][4][64]
constexpr int kRedS = kRedT + kMaxTiles * 2 * 256;   // float offset of [2][16][16]: shared tile
constexpr int kDred = kWaves * kPairsPerWave * 64;   // float offset of [16][16] (after h slices)
constexpr int kRegionFloats = kDred + 256;
static_assert(kRedS + 512 <= kRegionFloats, "phase regions");

struct DecodeArgs {
    const uint16_t *x, *wr;
    const float *bias;
    const u32x4 *w13;
    const void *s13;  // fp16 [G][2I][H/128] (INT4) or UE8M0 [G][2I][H/32] (FP4)
    const u32x4 *w2;
    const void *s2;   // fp16 [G][H][I/128] (INT4) or UE8M0 [G][H][I/32] (FP4)
    int E, k, ns, H, I;
    int kgi_mul;  // ceil(2^16 / (I/128)): pp / (I/128) = (pp * kgi_mul) >> 16 for pp < 2^16 / 32
    float routed_scale;
    float *logits;
    int32_t *topk_idx;
    float *topk_w;
    int32_t *offsets, *sorted_token, *row_of_slot;
    uint16_t *h, *out;
    int32_t *ws;
};

// LDS-only workgroup barrier: waits for this wave's LDS operations, not for
// its loads from global memory still in flight.
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void lds_sync_wave() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Workgroup barrier without a fence: the calling wave's LDS writes have
// completed (lgkmcnt) when `lds_writes`, nothing else is waited for.
__device__ __forceinline__ void raw_sync(bool lds_writes) {
    if (lds_writes) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void dma4(const void *g, void *lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void_t *)lds, 4, 0, 0);
}

template <typename T>
__device__ __forceinline__ void store_coherent(T *p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T load_coherent(const T *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave-wide wait until every one of the n 32-bit words at w[0..n) (n <= 256,
// four per lane) holds the tag, polling with device-coherent loads for at
// most kWaitTicks; on time-out the error word is raised.
// The four words of a lane are read as two 64-bit words, every one of them
// each time (w must have 256 readable words), so that one poll is one
// memory round trip.
__device__ void wait_tags(const uint32_t *w, int n, uint32_t tag, int32_t *err) {
    const int l = lane_id();
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    const uint64_t *w2 = (const uint64_t *)(w + 4 * l);
    for (;;) {
        const uint64_t a = load_coherent(w2), b = load_coherent(w2 + 1);
        const bool ok = (4 * l + 0 >= n || (uint32_t)a == tag) && (4 * l + 1 >= n || (uint32_t)(a >> 32) == tag) &&
                        (4 * l + 2 >= n || (uint32_t)b == tag) && (4 * l + 3 >= n || (uint32_t)(b >> 32) == tag);
        if (__all(ok)) return;
        if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
            if (l == 0) store_coherent(err, 1);
            return;
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

// The MFMA A operand whose row 0 is the 128-element vector at src (lane l
// holds k = 32*(l/16) + 8d + [0,8) of row l%16).  Every row reads the same
// vector: a row of the product depends only on the same row of A, and only
// row 0 is used.
__device__ __forceinline__ void a_row0(const uint16_t *src, int q, u32x4 (&av)[4]) {
#pragma unroll
    for (int d = 0; d < 4; ++d) av[d] = *(const u32x4 *)(src + 32 * q + 8 * d);
}

// LDS counters between the waves of one workgroup, without a workgroup
// barrier (the waves loading into LDS must not be waited for): a wave's LDS
// writes complete before it adds to the counter; the reader spins on it.
__device__ __forceinline__ void lds_signal(int *c) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    if (lane_id() == 0) __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_wait(int *c, int target, int32_t *err) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
        if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
            if (lane_id() == 0) store_coherent(err, 1);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
}

// sum_k a[k] * (code[k] + 136) over one 128-wide k group, plus the
// accumulator input c
__device__ __forceinline__ f32x4 mfma_group(const u32x4 (&av)[4], u32x4 w, f32x4 c) {
#pragma unroll
    for (int d = 0; d < 4; ++d) c = mfma16(__builtin_bit_cast(bf16x8, av[d]), unpack_codes(w[d]), c);
    return c;
}

// the same over FP4 codes w scaled by s (no offset term)
__device__ __forceinline__ f32x4 mfma_group_fp4(const u32x4 (&av)[4], u32x4 w, float s, f32x4 c) {
#pragma unroll
    for (int d = 0; d < 4; ++d) c = mfma16(__builtin_bit_cast(bf16x8, av[d]), fp4x8_to_bf16(w[d], s), c);
    return c;
}

__device__ __forceinline__ f32x4 mfma_offset(const u32x4 (&av)[4]) {
    bf16x8 bneg;
#pragma unroll
    for (int i = 0; i < 8; ++i) bneg[i] = __builtin_bit_cast(__bf16, kNeg136);
    f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < 4; ++d) c = mfma16(__builtin_bit_cast(bf16x8, av[d]), bneg, c);
    return c;
}

// h = silu(g) * u for the n columns held by lanes lo..lo+n-1 (lo, n even),
// stored as bf16 pairs (even lanes) at h_row[0..n) and, with the epoch tag
// in the upper half, as n/2 64-bit device-coherent words at htag[0..n/2).
__device__ __forceinline__ void store_h_cols(float g, float u, uint16_t *h_row, uint64_t *htag,
                                             uint32_t tag, int lo, int n) {
    const int l = lane_id();
    const float hv = silu_mul(g, u);
    const float hn = __shfl_down(hv, 1, kWave);
    if (l >= lo && l < lo + n && (l & 1) == 0) {
        const uint32_t pr = pack_bf16x2(hv, hn);
        *(uint32_t *)(h_row + (l - lo)) = pr;
        store_coherent(htag + ((l - lo) >> 1), ((uint64_t)tag << 32) | pr);
    }
}

// Q8 (W4A8, FP4 experts only): the expert GEMMs take x and h quantised to
// e4m3 with one power-of-two scale per 128 consecutive elements (the
// arithmetic of moe_act_quant_fp8); the quantised values are exact in bf16,
// so the bf16 matrix instructions multiply exactly them.  The router reads
// x as it is.
template <int FMT, int KG, int MAXT, bool Q8>
__device__ __forceinline__ void decode_body(DecodeArgs p) {
    static_assert(MAXT >= 1 && MAXT <= kMaxTiles, "tiles per workgroup");
    static_assert(!Q8 || FMT == kFmtFp4, "W4A8 takes FP4 experts");
    constexpr int HJ = KG / 4;    // H / 512: router words per lane
    constexpr int KGQ = KG / 4;   // k groups of a gate/up wave
    const int b = blockIdx.x, P = gridDim.x;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = lane_id(), m = l & 15, q = l >> 4;
    const int E = p.E, k = p.k, ns = p.ns, H = p.H, I = p.I;
    const int S = k + ns, KGI = I >> 7, NTI = I >> 4, NTH = H >> 4;
    const int npairs = S * KGI;
    int32_t *const ws = p.ws;
    uint64_t *const scores = (uint64_t *)(ws + kWsScores);  // copy r at scores + 512 r
    uint32_t *const done = (uint32_t *)(ws + kWsDone);
    uint64_t *const htag = (uint64_t *)(ws + kWsHtag);      // slot s at htag + s * I/2

    __shared__ u32x4 wdn[kMaxPairs + 1][kWave];  // + a slot for the loads past the last pair
    constexpr int kScaleDwords = scale_dwords<FMT>();
    constexpr int kScaleDmaPerWave = scale_dma_per_wave<FMT>();
    __shared__ __attribute__((aligned(16))) uint32_t sdl[kScaleDwords + 64];  // down scales
    __shared__ __attribute__((aligned(16))) float region[kRegionFloats];
    __shared__ float xneg[32];  // -136 * (sum of x over each 128-wide k group)
    __shared__ int sel_idx[8], slot_row[9], slot_g[9], g_lds[kWave];
    __shared__ float sel_w[9];
    __shared__ int tile_cnt[kMaxTiles];  // phase-2 counters between waves
    __shared__ int routed;               // wave 0 has written slot_row and sel_w
    uint16_t *const xs = (uint16_t *)region;
    float *const redT = region + kRedT;
    float *const redS = region + kRedS;
    uint16_t *const hsl = (uint16_t *)region;
    float *const dred = region + kDred;

    // ------------------------------------------------------------ phase 0
    // this call's epoch (workgroup 0 of the previous call advanced it) and
    // the error word (both loads in flight at once).  A raised error word is sticky: every
    // later call returns here without writing anything until the caller
    // zeroes the workspace, so no call can accept words that a workgroup of
    // a timed-out call wrote late.  (The decision is per wave: a wave that
    // returns while the others of its workgroup go on only makes them wait
    // out their bounded waits in a call that has already failed.)
    const int32_t err_word = load_coherent(ws + kWsErr);
    const uint32_t epoch = (uint32_t)load_coherent(ws + kWsEpoch);
    // the loads that need neither go out with them, so that the check costs
    // no round trip of its own before the router rows are requested: wave
    // 0's gate biases (it selects later), x, and the router rows of this
    // wave's expert
    // (in-bounds addresses, loaded by every lane and selected afterwards: a
    // load under a lane condition makes the compiler's count for the words
    // above it wait for nearly everything issued after them)
    float bs[4] = {0.f, 0.f, 0.f, 0.f};
    if (wave == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) bs[i] = p.bias[min(4 * l + i, E - 1)];
    }
    const bool xl = (int)threadIdx.x < (H >> 3);
    u32x4 xv0 = *(const u32x4 *)(p.x + 8 * min((int)threadIdx.x, (H >> 3) - 1));
    const int e_r = b + P * wave;
    const bool router_wave = wave < 4 && e_r < E;
    u32x4 xr[HJ], wrv[HJ];
    if (router_wave) {
#pragma unroll
        for (int j = 0; j < HJ; ++j) xr[j] = *(const u32x4 *)(p.x + 512 * j + 8 * l);
#pragma unroll
        for (int j = 0; j < HJ; ++j) wrv[j] = *(const u32x4 *)(p.wr + (size_t)e_r * H + 512 * j + 8 * l);
    }
    // the router waves' dot product needs every row it requested; the check
    // follows it, so it waits for nothing more on their path.  Nothing is
    // stored before the check.
    float rv = 0.0f;
    if (router_wave) rv = route::router_dot<HJ>(xr, wrv);
    if (__builtin_amdgcn_readfirstlane(err_word) != 0) return;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (4 * l + i >= E) bs[i] = 0.0f;
    if (!xl) xv0 = u32x4{0u, 0u, 0u, 0u};
    const uint32_t tag = epoch + 1u;
    // this workgroup has read the epoch: workgroup 0 may advance it once
    // every flag is up
    if (wave == 0 && l == 0) store_coherent(done + b, tag);
    if (router_wave) {
        if (l == 0) store_coherent(p.logits + e_r, rv);
        if (l < kReplicas)
            store_coherent(scores + 512 * l + e_r,
                           ((uint64_t)tag << 32) | __float_as_uint(route::sigmoid_f32(rv)));
    }
    // the shared expert's gate/up tile b/2, h columns 8*(b%2)..+8 of its 16
    // over all of K, for b < 2*I/16: the lanes that hold those weight rows
    // load their half of every 1 KB block.  K group kg goes to wave
    // 1 + kg % kShWaves.  Those waves load nothing else before phase 2; wave
    // 0 polls the scores next and must have no load of its own in flight.
    constexpr int SHK = (KG + kShWaves - 1) / kShWaves;  // k groups per wave
    const bool shared_tile = ns && b < 2 * NTI;
    const int sh_tile = b >> 1, sh_lo = 8 * (b & 1);  // tile, first column
    const bool shw = shared_tile && wave >= 1 && wave <= kShWaves;
    const bool sh_lane = (m & 8) == sh_lo;            // lane holds one of the 8 rows
    u32x4 pg[SHK], pu[SHK];
    uint16_t psg[SHK], psu[SHK];
    {
        const u32x4 *pw13 = p.w13 + (size_t)(E * 2 * NTI + sh_tile) * KG * kWave + l;
        const uint16_t *ps13 = (const uint16_t *)p.s13 + ((size_t)E * 2 * I + 16 * sh_tile + m) * KG;
        const uint8_t *ps13b = (const uint8_t *)p.s13 + ((size_t)E * 2 * I + 16 * sh_tile + m) * (H >> 5) + q;
        const size_t up13 = (size_t)NTI * KG * kWave;  // gate -> up rows, in 16-byte words
#pragma unroll
        for (int i = 0; i < SHK; ++i) {
            pg[i] = pu[i] = u32x4{0u, 0u, 0u, 0u};
            psg[i] = psu[i] = 0;
            const int kg = (wave - 1) + kShWaves * i;
            if (shw && kg < KG && sh_lane) {
                pg[i] = pw13[(size_t)kg * kWave];
                pu[i] = pw13[up13 + (size_t)kg * kWave];
                if constexpr (FMT == kFmtInt4) {
                    psg[i] = ps13[kg];
                    psu[i] = ps13[(size_t)I * KG + kg];
                } else {  // the scale byte of this lane's 32-wide block
                    psg[i] = ps13b[kg * 4];
                    psu[i] = ps13b[(size_t)I * (H >> 5) + kg * 4];
                }
            }
        }
    }
    if constexpr (Q8) {
        // each 128-element block of x: sixteen lanes of eight elements (H/8
        // lanes hold x, a multiple of sixteen)
        float xf[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xf[2 * i] = __uint_as_float(xv0[i] << 16);
            xf[2 * i + 1] = __uint_as_float(xv0[i] & 0xFFFF0000u);
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(xf[i]));
#pragma unroll
        for (int d = 8; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, kWave));
        const int Ex = act_scale_code(amax);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            xv0[i] = pack_bf16x2(fp8_roundtrip(xf[2 * i], Ex), fp8_roundtrip(xf[2 * i + 1], Ex));
    }
    if (xl) *(u32x4 *)(xs + 8 * threadIdx.x) = xv0;
    if (threadIdx.x < kMaxTiles) tile_cnt[threadIdx.x] = 0;
    if (threadIdx.x == 0) routed = 0;
    lds_sync();
    // the code-offset term of the routed gate/up tiles, once per k group:
    // sixteen lanes add eight consecutive elements each, then pairwise
    if ((int)threadIdx.x < KG * 16) {
        float sx = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sx += bf16lo_to_f32(xv0[i]);
            sx += bf16hi_to_f32(xv0[i]);
        }
#pragma unroll
        for (int d = 8; d >= 1; d >>= 1) sx += __shfl_xor(sx, d, kWave);
        if ((threadIdx.x & 15) == 0) xneg[threadIdx.x >> 4] = -136.0f * sx;
    }
    // the shared expert's down rows of this workgroup's columns (pairs
    // k*KGI.., group E) need no routing: loaded into LDS now
    if (ns && b < NTH && wave >= kDmaWave0) {
#pragma unroll
        for (int i = 0; i < kShDmaPerWave; ++i) {
            const int kg = (wave - kDmaWave0) + kDmaWaves * i;
            const bool real = kg < KGI;
            const u32x4 *src = real ? p.w2 + ((size_t)(E * NTH + b) * KGI + kg) * kWave + l : p.w2 + l;
            dma16(src, &wdn[real ? k * KGI + kg : kMaxPairs][0]);
        }
    }
    // this wave's k groups of the shared tile (row 0 of the MFMA tiles),
    // computed while wave 0 selects; every wave writes its slot of redS
    auto shared_part = [&]() {
        float tg = 0.0f, tu = 0.0f;
        if (shw) {
#pragma unroll
            for (int i = 0; i < SHK; ++i) {
                const int kg = (wave - 1) + kShWaves * i;
                if (kg < KG) {
                    u32x4 av[4];
                    a_row0(xs + kg * 128, q, av);
                    if constexpr (FMT == kFmtInt4) {
                        const f32x4 nc = mfma_offset(av);
                        tg = __builtin_fmaf(half_bits_to_f32(psg[i]), mfma_group(av, pg[i], nc)[0], tg);
                        tu = __builtin_fmaf(half_bits_to_f32(psu[i]), mfma_group(av, pu[i], nc)[0], tu);
                    } else {
                        const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
                        tg += mfma_group_fp4(av, pg[i], ue8m0_to_f32(psg[i]), z)[0];
                        tu += mfma_group_fp4(av, pu[i], ue8m0_to_f32(psu[i]), z)[0];
                    }
                }
            }
        }
        if (l < 16) {
            redS[wave * 16 + l] = tg;
            redS[256 + wave * 16 + l] = tu;
        }
    };
    // ------------------------------------------------------------ phase 1
    shared_part();  // wave 0 has no share: it writes zeros and polls
    // the E tagged scores, four per lane, and the chosen expert of lane j < k
    float sc[4] = {0.f, 0.f, 0.f, 0.f};
    int es = 0;
    if (wave == 0) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        // every lane reads its four words each time (a copy has 512), so
        // that one poll is one memory round trip
        const uint64_t *mine = scores + 512 * (b % kReplicas) + 4 * l;
        for (;;) {
            uint64_t v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = load_coherent(mine + i);
            bool ok = true;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ok = ok & (4 * l + i >= E || (uint32_t)(v[i] >> 32) == tag);
                sc[i] = 4 * l + i < E ? __uint_as_float((uint32_t)v[i]) : 0.0f;
            }
            if (__all(ok)) break;
            if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
                if (l == 0) store_coherent(ws + kWsErr, 1);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        // the experts only: the phase-2 loads need nothing else, so the
        // routing weights and the permuted rows come after they are issued
        es = route::select_experts(sc, bs, E, k);
        if (l < k) slot_g[l] = min(max(es, 0), E - 1);
        if (l == 0) slot_g[k] = E;  // the shared expert (when there is one)
        if (l > k && l < 9) slot_g[l] = 0;  // unused entries: defined values
    }
    // no fence: the waves loading into LDS must not wait for those loads here
    raw_sync(true);
    // the shared half tile's h, from the partials of waves 1..kShWaves (in
    // LDS since the barrier above).  Written by wave 0 once its phase-2 loads
    // are in flight: a wave that has just issued loads into LDS would first
    // wait for them to land (its LDS reads might read what they write), and
    // every workgroup's down product waits for this slot's h.
    auto finish_shared = [&]() {
        float g = 0.0f, u = 0.0f;
        if (l < 16)
            for (int w = 1; w <= kShWaves; ++w) {
                g += redS[w * 16 + l];
                u += redS[256 + w * 16 + l];
            }
        store_h_cols(g, u, p.h + (size_t)k * I + 16 * sh_tile + sh_lo,
                     htag + (size_t)k * (I >> 1) + 8 * sh_tile + (sh_lo >> 1), tag, sh_lo, 8);
    };
    bool shared_open = wave == 0 && shared_tile;
    // the rest of the routing (wave 0, with its phase-2 loads in flight):
    // the weights and, per routed slot, its permuted row (the number of
    // chosen experts below its expert: the choice has k distinct experts;
    // the shared slot comes after them); workgroup 0 writes the routing
    // outputs.  The tile finalizers wait for it (slot_row), phase 3 reads
    // sel_w after a workgroup barrier.
    auto finish_routing = [&]() {
        route::route_weights(sc, es, k, p.routed_scale, sel_idx, sel_w);
        int r = 0;
        for (int j = 0; j < k; ++j) r += __builtin_amdgcn_readlane(es, j) < es;
        if (l < k) slot_row[l] = r;
        if (l == 0) {
            slot_row[k] = k;
            sel_w[k] = 1.0f;
        }
        if (l > k && l < 9) {
            slot_row[l] = 0;
            sel_w[l] = 0.0f;
        }
        lds_sync_wave();
        if (b == 0) {
            if (l < k) {
                p.topk_idx[l] = es;
                p.topk_w[l] = sel_w[l];
            }
            route::permute_small(sel_idx, 1, E, k, ns, g_lds, p.offsets, p.sorted_token, p.row_of_slot);
        }
        lds_signal(&routed);
    };
    bool routing_open = wave == 0;

    // ------------------------------------------------------------ phase 2
    const int nroute = k * NTI;
    if (wave < 4 * MAXT) {
        // gate/up wave: tile gt of this workgroup, k groups [kq*KGQ, +KGQ)
        const int gt = wave >> 2, kq = wave & 3;
        const int j = b + P * gt;
        if (j < nroute) {
            const int s = j / NTI, c = j - s * NTI;
            const int e = __builtin_amdgcn_readfirstlane(slot_g[s]);
            // scales of row 16c+m (gate) and I+16c+m (up) for the wave's k
            // groups first (the k groups are then finished as their weights
            // land), then the weights
            // (FP4: dword u of sgb / sub holds the four block scales of k
            // group kq*KGQ + u; this lane's is byte q)
            u32x4 sgv = u32x4{0u, 0u, 0u, 0u}, suv = sgv;
            uint32_t sgb[KGQ], sub[KGQ];
            if constexpr (FMT == kFmtInt4) {
                const uint16_t *sp = (const uint16_t *)p.s13 + ((size_t)e * 2 * I + 16 * c + m) * KG + kq * KGQ;
                if constexpr (KGQ == 8) {
                    sgv = *(const u32x4 *)sp;
                    suv = *(const u32x4 *)(sp + (size_t)I * KG);
                } else {
                    const uint2 a0 = *(const uint2 *)sp, a1 = *(const uint2 *)(sp + (size_t)I * KG);
                    sgv = u32x4{a0.x, a0.y, 0u, 0u};
                    suv = u32x4{a1.x, a1.y, 0u, 0u};
                }
            } else {
                const uint8_t *sb = (const uint8_t *)p.s13 + ((size_t)e * 2 * I + 16 * c + m) * (H >> 5) + kq * KGQ * 4;
                const size_t upb = (size_t)I * (H >> 5);
#pragma unroll
                for (int j4 = 0; j4 < KGQ / 4; ++j4) {
                    const u32x4 g4 = *(const u32x4 *)(sb + 16 * j4), u4 = *(const u32x4 *)(sb + upb + 16 * j4);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        sgb[4 * j4 + t] = g4[t];
                        sub[4 * j4 + t] = u4[t];
                    }
                }
            }
            u32x4 wg[KGQ], wu[KGQ];
#pragma unroll
            for (int u = 0; u < KGQ; ++u) {
                const int kg = kq * KGQ + u;
                wg[u] = p.w13[((size_t)(e * 2 * NTI + c) * KG + kg) * kWave + l];
                wu[u] = p.w13[((size_t)(e * 2 * NTI + NTI + c) * KG + kg) * kWave + l];
            }
            __builtin_amdgcn_sched_barrier(0);  // every load issued before the first wait
            if (shared_open) {
                finish_shared();
                shared_open = false;
            }
            if (routing_open) {
                finish_routing();
                routing_open = false;
            }
            // tile row 0 (lanes 0..15, element 0) is the token's; the
            // -136 * sum(x) term comes from xneg
            float ag = 0.0f, au = 0.0f;
#pragma unroll
            for (int u = 0; u < KGQ; ++u) {
                u32x4 av[4];
                a_row0(xs + (kq * KGQ + u) * 128, q, av);
                const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
                if constexpr (FMT == kFmtInt4) {
                    const f32x4 tg = mfma_group(av, wg[u], zero);
                    const f32x4 tu = mfma_group(av, wu[u], zero);
                    const float nc = xneg[kq * KGQ + u];
                    const float sg = half_bits_to_f32((uint16_t)(sgv[u >> 1] >> (16 * (u & 1))));
                    const float su = half_bits_to_f32((uint16_t)(suv[u >> 1] >> (16 * (u & 1))));
                    ag = __builtin_fmaf(sg, tg[0] + nc, ag);
                    au = __builtin_fmaf(su, tu[0] + nc, au);
                } else {
                    const float sg = ue8m0_to_f32((sgb[u] >> (8 * q)) & 0xFFu);
                    const float su = ue8m0_to_f32((sub[u] >> (8 * q)) & 0xFFu);
                    ag += mfma_group_fp4(av, wg[u], sg, zero)[0];
                    au += mfma_group_fp4(av, wu[u], su, zero)[0];
                }
            }
            // every lane stores (only lanes 0..15 carry tile row 0): a store
            // under a lane condition lets the compiler sink the scale loads
            // and their arithmetic past the last MFMA
            redT[((gt * 2) * 4 + kq) * 64 + l] = ag;
            redT[((gt * 2 + 1) * 4 + kq) * 64 + l] = au;
            lds_signal(&tile_cnt[gt]);
        }
    }
    if (wave >= kDmaWave0 && b < NTH) {
        // the slots' groups, read from LDS before the first load into LDS
        int gsl[9];
#pragma unroll
        for (int i = 0; i < 9; ++i) gsl[i] = __builtin_amdgcn_readfirstlane(slot_g[i]);
        // down rows of output columns 16b.. for routed pair pp = (slot
        // pp / KGI, k group pp % KGI) into wdn[pp]; a fixed number per wave,
        // the loads past the last pair re-read the first block into a spare
        // slot
#pragma unroll
        for (int i = 0; i < kDmaPerWave; ++i) {
            const int pp = (wave - kDmaWave0) + kDmaWaves * i;
            const bool real = pp < k * KGI;
            const int ppc = real ? pp : 0;
            const int s = ppc / KGI, kg = ppc - s * KGI;
            int g = gsl[0];
#pragma unroll
            for (int jj = 1; jj < 9; ++jj) g = s == jj ? gsl[jj] : g;
            const u32x4 *src = real ? p.w2 + ((size_t)(g * NTH + b) * KGI + kg) * kWave + l : p.w2 + l;
            dma16(src, &wdn[real ? pp : kMaxPairs][0]);
        }
        // their scales: slot s holds 16 rows x KGI fp16 (INT4) or 16 rows x
        // 4*KGI UE8M0 bytes (FP4) = SDK*KGI dwords, contiguous in w_scales;
        // dword d of the workgroup's list lands at sdl[d]; lanes past the
        // list re-read the slot's first dword into the spare tail
        constexpr int SDK = scale_dwords_per_kg<FMT>();
        const int sdw = SDK * KGI;
#pragma unroll
        for (int i = 0; i < kScaleDmaPerWave; ++i) {
            const int d0 = 64 * ((wave - kDmaWave0) + kDmaWaves * i);
            const int d = d0 + l;
            const bool real = d < npairs * SDK;
            const int dc = real ? d : 0;
            const int s = dc / sdw, o = dc - s * sdw;
            int g = gsl[0];
#pragma unroll
            for (int jj = 1; jj < 9; ++jj) g = s == jj ? gsl[jj] : g;
            const uint32_t *src =
                FMT == kFmtInt4 ? (const uint32_t *)((const uint16_t *)p.s2 + ((size_t)g * H + 16 * b) * KGI) + o
                                : (const uint32_t *)((const uint8_t *)p.s2 + ((size_t)g * H + 16 * b) * (I >> 5)) + o;
            // an instruction that starts past the list writes the spare tail;
            // one that starts inside writes its 64 dwords in place (the tail
            // of the array absorbs lanes past the list)
            dma4(src, &sdl[d0 < npairs * SDK ? d0 : kScaleDwords]);
        }
    }
    if (shared_open) finish_shared();  // wave 0 had no routed tile
    if (routing_open) finish_routing();
    // finalizers: the first wave of each routed tile adds the tile's four k
    // quarters in order and writes its h.  The waves loading into LDS are
    // not waited for.
    if (wave < 4 * MAXT && (wave & 3) == 0) {
        const int gt = wave >> 2;
        const int j = b + P * gt;
        if (j < nroute) {
            lds_wait(&tile_cnt[gt], 4, ws + kWsErr);
            lds_wait(&routed, 1, ws + kWsErr);  // slot_row
            const int s = j / NTI, c = j - s * NTI;
            float g = 0.0f, u = 0.0f;
            if (l < 16)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    g += redT[((gt * 2) * 4 + w) * 64 + l];
                    u += redT[((gt * 2 + 1) * 4 + w) * 64 + l];
                }
            store_h_cols(g, u, p.h + (size_t)slot_row[s] * I + 16 * c, htag + (size_t)s * (I >> 1) + 8 * c,
                         tag, 0, 16);
        }
    }

    // ------------------------------------------------------------ phase 3
    if (b < NTH) {
        // the pairs of this wave, pp = wave + 16 i: slot and k group before
        // anything is waited for (pairs past the last re-read the last one,
        // with weight 0)
        int pkg[kPairsPerWave], pslot[kPairsPerWave];
#pragma unroll
        for (int i = 0; i < kPairsPerWave; ++i) {
            const int pp = min(wave + kWaves * i, npairs - 1);
            const int s = (pp * p.kgi_mul) >> 16;
            pslot[i] = s;
            pkg[i] = pp - s * KGI;
        }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads into LDS have landed
        lds_sync();                     // every wave's have; phase 2 is over
        // the routing weights: wave 0 wrote them in phase 2
        float pw[kPairsPerWave];
#pragma unroll
        for (int i = 0; i < kPairsPerWave; ++i) pw[i] = wave + kWaves * i < npairs ? sel_w[pslot[i]] : 0.0f;
        // the pairs' h slices (columns 2l, 2l+1 of the k group), polled until
        // every word carries this call's tag.  The first read is an ordinary
        // load, which the compute units of one XCD can share through its L2
        // (every workgroup reads all of h); a word it finds with an older tag
        // (not yet written, or an older line cached) is read again with
        // device-coherent loads until it carries this call's.  While the
        // first read is in flight the wave unpacks the down rows of its first
        // kPre pairs (the unpacking is most of the VALU work of this phase).
        constexpr int kPre = 5;
        uint64_t hv[kPairsPerWave];
        const uint64_t *hsrc[kPairsPerWave];
#pragma unroll
        for (int i = 0; i < kPairsPerWave; ++i) hsrc[i] = htag + (size_t)pslot[i] * (I >> 1) + pkg[i] * 64 + l;
        auto poll = [&]() {
#pragma unroll
            for (int i = 0; i < kPairsPerWave; ++i) hv[i] = load_coherent(hsrc[i]);
        };
        auto all_tagged = [&]() {
            bool ok = true;
#pragma unroll
            for (int i = 0; i < kPairsPerWave; ++i) ok = ok & ((uint32_t)(hv[i] >> 32) == tag);
            return __all(ok);
        };
#pragma unroll
        for (int i = 0; i < kPairsPerWave; ++i) hv[i] = *hsrc[i];
        // FP4: this lane's block scale of pair i, row m, block 4*kg + q
        const uint8_t *sdl8 = (const uint8_t *)sdl + m * (I >> 5) + q;
        auto fp4_scale = [&](int i) { return ue8m0_to_f32(sdl8[pslot[i] * 16 * (I >> 5) + pkg[i] * 4]); };
        bf16x8 wu[kPre][4];
#pragma unroll
        for (int i = 0; i < kPre; ++i) {
            const u32x4 w = wdn[min(wave + kWaves * i, npairs - 1)][l];
            const float si = FMT == kFmtFp4 ? fp4_scale(i) : 0.0f;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                wu[i][d] = FMT == kFmtInt4 ? unpack_codes(w[d]) : fp4x8_to_bf16(w[d], si);
                asm volatile("" : "+v"(wu[i][d]));  // computed here, before the poll is waited for
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (!all_tagged()) {
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            for (;;) {
                __builtin_amdgcn_s_sleep(2);
                poll();
                if (all_tagged()) break;
                if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
                    if (l == 0) store_coherent(ws + kWsErr, 1);
                    break;
                }
            }
        }
        // Q8: each pair's 128 h values are one quantisation block (columns
        // 128 kg.. of its row), two per lane; their maxima |h| are taken on
        // the bit patterns (non-negative floats order as their bits) with
        // the wave-wide maximum of the routing code, every pair's at once
        uint32_t amx[kPairsPerWave];
        if constexpr (Q8) {
#pragma unroll
            for (int i = 0; i < kPairsPerWave; ++i) {
                const uint32_t pr = (uint32_t)hv[i];
                amx[i] = max((pr << 16) & 0x7FFFFFFFu, pr & 0x7FFF0000u);
            }
#pragma unroll
            for (int i = 0; i < kPairsPerWave; ++i) amx[i] = route::wave_max32(amx[i]);
        }
#pragma unroll
        for (int i = 0; i < kPairsPerWave; ++i) {
            uint32_t pr = (uint32_t)hv[i];
            if constexpr (Q8) {
                const int Eh = act_scale_code(__uint_as_float(amx[i]));
                pr = pack_bf16x2(fp8_roundtrip(__uint_as_float(pr << 16), Eh),
                                 fp8_roundtrip(__uint_as_float(pr & 0xFFFF0000u), Eh));
            }
            *(uint32_t *)(hsl + (wave * kPairsPerWave + i) * 128 + 2 * l) = pr;
        }
        lds_sync_wave();
        // per pair: -136 * sum(h) from one MFMA whose rows 0..3 hold the four
        // 32-wide chunks of the slice (B = -136), then the four MFMAs of the
        // product with that in row 0 of the accumulator.  No branches: the
        // pairs' MFMA chains interleave.
        bf16x8 bneg;
#pragma unroll
        for (int j = 0; j < 8; ++j) bneg[j] = __builtin_bit_cast(__bf16, kNeg136);
        const uint16_t *sdl16 = (const uint16_t *)sdl + m * KGI;  // row m of each slot's scales
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < kPairsPerWave; ++i) {
            const uint16_t *hs = hsl + (wave * kPairsPerWave + i) * 128;
            u32x4 av[4];
            a_row0(hs, q, av);
            if constexpr (FMT == kFmtFp4) {  // scales folded into the weights, no offset term
                f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
                if (i < kPre) {
#pragma unroll
                    for (int d = 0; d < 4; ++d) t = mfma16(__builtin_bit_cast(bf16x8, av[d]), wu[i][d], t);
                } else {
                    t = mfma_group_fp4(av, wdn[min(wave + kWaves * i, npairs - 1)][l], fp4_scale(i), t);
                }
                acc = __builtin_fmaf(pw[i], t[0], acc);
                continue;
            }
            const u32x4 a4 = *(const u32x4 *)(hs + 32 * min(m, 3) + 8 * q);
            const f32x4 c4 = mfma16(__builtin_bit_cast(bf16x8, a4), bneg, f32x4{0.f, 0.f, 0.f, 0.f});
            const float nc = (c4[0] + c4[1]) + (c4[2] + c4[3]);
            f32x4 t = f32x4{nc, 0.f, 0.f, 0.f};
            if (i < kPre) {
#pragma unroll
                for (int d = 0; d < 4; ++d) t = mfma16(__builtin_bit_cast(bf16x8, av[d]), wu[i][d], t);
            } else {
                t = mfma_group(av, wdn[min(wave + kWaves * i, npairs - 1)][l], t);
            }
            const uint16_t sraw = sdl16[pslot[i] * 16 * KGI + pkg[i]];
            acc = __builtin_fmaf(pw[i], half_bits_to_f32(sraw) * t[0], acc);
        }
        if (l < 16) dred[wave * 16 + l] = acc;
        lds_sync();
        if (wave == 0 && l < 16) {
            float v = 0.0f;
            for (int w = 0; w < kWaves; ++w) v += dred[w * 16 + l];
            p.out[16 * b + l] = f32_to_bf16(v);
        }
    }
    // workgroup 0, last: once every workgroup has read the epoch (its flag is
    // up), the next call's epoch can be published
    // (not after a wait of this call timed out: the error word then stops
    // every later call before it reads the epoch)
    if (b == 0 && wave == 0) {
        wait_tags(done, P, tag, ws + kWsErr);
        if (l == 0 && load_coherent(ws + kWsErr) == 0) store_coherent(ws + kWsEpoch, (int32_t)tag);
    }
}

template <int KG, int MAXT>
__global__ __launch_bounds__(1024) void k_decode_token(DecodeArgs p) {
    decode_body<kFmtInt4, KG, MAXT, false>(p);
}

template <int KG, int MAXT>
__global__ __launch_bounds__(1024) void k_mxfp4_decode_token(DecodeArgs p) {
    decode_body<kFmtFp4, KG, MAXT, false>(p);
}

template <int KG, int MAXT>
__global__ __launch_bounds__(1024) void k_w4a8_decode_token(DecodeArgs p) {
    decode_body<kFmtFp4, KG, MAXT, true>(p);
}

// ---------------------------------------------------------------- host
struct DecodePlan {
    int grid;  // one workgroup per CU
    int kg, maxt;
};

// Compute units of the current device (cached per device).
int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cus[dev] = n;
    }
    return cus[dev];
}

// Limits of the shape alone (no device query).
moe_status decode_shape(const moe_layer_desc *d) {
    MOE_TRY(check_desc(d));
    const int H = d->hidden, I = d->inter, S = d->top_k + d->n_shared;
    if (H != 2048 && H != 4096) return MOE_ERR_UNSUPPORTED;
    if (S * (I / 128) > kMaxPairs || I / 16 > 256) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// Limits the current device adds: every workgroup resident at once, one per
// CU, with enough of them for the output columns and the tiles.
moe_status decode_plan(const moe_layer_desc *d, DecodePlan &pl) {
    MOE_TRY(decode_shape(d));
    const int H = d->hidden, I = d->inter;
    const int cus = device_cus();
    if (cus <= 0) return MOE_ERR_DEVICE;
    if (cus > kMaxGrid) return MOE_ERR_UNSUPPORTED;  // one score / done slot per workgroup
    if (cus < H / 16) return MOE_ERR_UNSUPPORTED;  // one workgroup per 16 output columns
    if (d->n_shared && cus < 2 * (I / 16)) return MOE_ERR_UNSUPPORTED;  // half a shared tile each
    if (cus * 4 < d->n_routed) return MOE_ERR_UNSUPPORTED;  // router waves 0..3
    const int tiles = d->top_k * (I / 16);
    const int maxt = (tiles + cus - 1) / cus;
    if (maxt > kMaxTiles) return MOE_ERR_UNSUPPORTED;
    pl.grid = cus;
    pl.kg = H / 128;
    pl.maxt = maxt;
    return MOE_OK;
}

template <int FMT, int KG, bool Q8>
void launch_decode(int maxt, int grid, const DecodeArgs &a, hipStream_t st) {
    auto k1 = FMT == kFmtInt4 ? k_decode_token<KG, 1> : Q8 ? k_w4a8_decode_token<KG, 1> : k_mxfp4_decode_token<KG, 1>;
    auto k2 = FMT == kFmtInt4 ? k_decode_token<KG, 2> : Q8 ? k_w4a8_decode_token<KG, 2> : k_mxfp4_decode_token<KG, 2>;
    auto k3 = FMT == kFmtInt4 ? k_decode_token<KG, 3> : Q8 ? k_w4a8_decode_token<KG, 3> : k_mxfp4_decode_token<KG, 3>;
    hipLaunchKernelGGL(maxt == 1 ? k1 : maxt == 2 ? k2 : k3, dim3(grid), dim3(1024), 0, st, a);
}

template <int FMT, bool Q8 = false>
moe_status decode_entry(const moe_layer_desc *desc, const uint16_t *x, const uint16_t *w_router,
                        const float *gate_bias, const uint8_t *w13_packed, const void *w13_scales,
                        const uint8_t *w2_packed, const void *w2_scales, float *logits, int32_t *topk_idx,
                        float *topk_w, int32_t *group_offsets, int32_t *sorted_token, int32_t *row_of_slot,
                        uint16_t *h, uint16_t *out, int32_t *workspace, void *stream) {
    MOE_TRY(decode_shape(desc));
    if (!x || !w_router || !gate_bias || !w13_packed || !w13_scales || !w2_packed || !w2_scales ||
        !logits || !topk_idx || !topk_w || !group_offsets || !sorted_token || !row_of_slot || !h ||
        !out || !workspace)
        return MOE_ERR_NULL;
    if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(gate_bias, 4) || !aligned(w13_packed, 16) ||
        !aligned(w13_scales, 16) || !aligned(w2_packed, 16) || !aligned(w2_scales, 4) ||
        !aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4) ||
        !aligned(group_offsets, 4) || !aligned(sorted_token, 4) || !aligned(row_of_slot, 4) ||
        !aligned(h, 16) || !aligned(out, 16) || !aligned(workspace, 16))
        return MOE_ERR_ALIGN;
    DecodePlan pl;
    MOE_TRY(decode_plan(desc, pl));
    const int kgi = desc->inter / 128;
    DecodeArgs a{x, w_router, gate_bias, (const u32x4 *)w13_packed, w13_scales, (const u32x4 *)w2_packed,
                 w2_scales, desc->n_routed, desc->top_k, desc->n_shared, desc->hidden, desc->inter,
                 (65536 + kgi - 1) / kgi, desc->routed_scale, logits, topk_idx, topk_w, group_offsets, sorted_token, row_of_slot,
                 h, out, workspace};
    hipStream_t st = (hipStream_t)stream;
    if (pl.kg == 32)
        launch_decode<FMT, 32, Q8>(pl.maxt, pl.grid, a, st);
    else
        launch_decode<FMT, 16, Q8>(pl.maxt, pl.grid, a, st);
    return launch_status();
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_w4a16_decode_token_supported(const moe_layer_desc *desc) {
    DecodePlan pl;
    return decode_plan(desc, pl);
}

extern "C" moe_status moe_w4a16_decode_token(
    const moe_layer_desc *desc, const uint16_t *x, const uint16_t *w_router, const float *gate_bias,
    const uint8_t *w13_packed, const uint16_t *w13_scales, const uint8_t *w2_packed,
    const uint16_t *w2_scales, float *logits, int32_t *topk_idx, float *topk_w, int32_t *group_offsets,
    int32_t *sorted_token, int32_t *row_of_slot, uint16_t *h, uint16_t *out, int32_t *workspace,
    void *stream) {
    return decode_entry<kFmtInt4>(desc, x, w_router, gate_bias, w13_packed, w13_scales, w2_packed, w2_scales,
                                  logits, topk_idx, topk_w, group_offsets, sorted_token, row_of_slot, h, out,
                                  workspace, stream);
}

extern "C" moe_status moe_mxfp4_decode_token(
    const moe_layer_desc *desc, const uint16_t *x, const uint16_t *w_router, const float *gate_bias,
    const uint8_t *w13_packed, const uint8_t *w13_scales, const uint8_t *w2_packed,
    const uint8_t *w2_scales, float *logits, int32_t *topk_idx, float *topk_w, int32_t *group_offsets,
    int32_t *sorted_token, int32_t *row_of_slot, uint16_t *h, uint16_t *out, int32_t *workspace,
    void *stream) {
    return decode_entry<kFmtFp4>(desc, x, w_router, gate_bias, w13_packed, w13_scales, w2_packed, w2_scales,
                                 logits, topk_idx, topk_w, group_offsets, sorted_token, row_of_slot, h, out,
                                 workspace, stream);
}

extern "C" moe_status moe_w4a8_decode_token(
    const moe_layer_desc *desc, const uint16_t *x, const uint16_t *w_router, const float *gate_bias,
    const uint8_t *w13_packed, const uint8_t *w13_scales, const uint8_t *w2_packed,
    const uint8_t *w2_scales, float *logits, int32_t *topk_idx, float *topk_w, int32_t *group_offsets,
    int32_t *sorted_token, int32_t *row_of_slot, uint16_t *h, uint16_t *out, int32_t *workspace,
    void *stream) {
    return decode_entry<kFmtFp4, true>(desc, x, w_router, gate_bias, w13_packed, w13_scales, w2_packed,
                                       w2_scales, logits, topk_idx, topk_w, group_offsets, sorted_token,
                                       row_of_slot, h, out, workspace, stream);
}
