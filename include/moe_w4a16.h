/*
 * moe_w4a16.h -- C ABI of the MI355X (gfx950) W4A16 routed-expert MoE layer.
 *
 * The layer is the MoE block of a DeepSeek-V4-Flash-style decoder: 256 routed
 * experts with six active per token and one always-on shared expert
 * ("DeepSeek V4 Flash serving hardware", 01, "Sparse architecture"), hidden
 * size 4096, routed experts stored as symmetric INT4 with one scale per 128
 * input elements and an FP32 gate bias (model card
 * "canada-quant/DeepSeek-V4-Flash-W4A16-FP8-MTP", "Architecture & precision"
 * and "Component precisions").  The weights are dequantised in registers and
 * multiplied with 16-bit activations, the weight-only scheme of
 * "Throughputmaxxing: DeepSeek-V4-Flash on Isambard-AI", "A pass through the
 * model".
 *
 * One forward pass is five calls on one stream:
 *     moe_route -> moe_permute -> moe_w4a16_grouped_gemm (gate/up, SwiGLU)
 *               -> moe_w4a16_grouped_gemm (down) -> moe_combine
 * (moe_route_permute does the first two in one call; for small batches
 * moe_w4a16_down_combine does the last two; for one token
 * moe_w4a16_decode_token does all of them.)
 *
 * Conventions for every entry point:
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise.
 *     The caller allocates and owns all memory; the library allocates and
 *     frees nothing and keeps no state between calls.
 *   - bf16 tensors are passed as uint16_t bit patterns, fp16 scales likewise.
 *   - All arguments are checked on the host before anything is enqueued; on
 *     an error nothing is enqueued and the status says why.  T == 0 returns
 *     MOE_OK with nothing enqueued.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream).  The library never synchronises.  Faults inside a
 *     kernel surface at the caller's next synchronisation.
 *   - A launch failure reported by the runtime returns MOE_ERR_LAUNCH.
 *   - Calls on distinct streams with distinct buffers may run concurrently.
 *   - Scratch memory comes from the caller: moe_permute and
 *     moe_route_permute take a workspace of moe_workspace_bytes(desc, T)
 *     bytes, the one-launch decode step one of MOE_DECODE_WORKSPACE_BYTES.
 *     The grouped GEMMs, the combine and the row sums need none and take no
 *     workspace argument.
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,        /* a required pointer is NULL                         */
    MOE_ERR_SHAPE = 2,       /* a size violates the limits stated below           */
    MOE_ERR_UNSUPPORTED = 3, /* a mode this build does not implement              */
    MOE_ERR_ALIGN = 4,       /* a pointer lacks the stated alignment              */
    MOE_ERR_LAUNCH = 5,      /* the HIP runtime rejected a kernel launch          */
    MOE_ERR_DEVICE = 6,      /* no usable gfx950 device is current                */
    MOE_ERR_WORKSPACE = 7    /* the workspace is smaller than moe_workspace_bytes */
} moe_status;

typedef enum moe_act {
    MOE_ACT_NONE = 0,   /* out = A . W^T                                           */
    MOE_ACT_SWIGLU = 1  /* W rows [0,N/2) = gate, [N/2,N) = up:                     */
                        /* out[:, n] = silu(gate_n) * up_n, N/2 columns            */
} moe_act;

/* Shape of one MoE layer.  Limits checked by every call:
 *   hidden     H: 512, 1024, 2048 or 4096 (multiple of 512 for the router's
 *                 64-lane order)
 *   inter      I: multiple of 128 with I/128 in {1,2,3,4,6,8,12,16,24,32}
 *   n_routed   E: 1..256
 *   top_k      k: 1..8 and k <= E
 *   n_shared    : 0 or 1 (the shared expert is group E)
 *   group_size  : 128 (scale group along the input dimension)
 *   routed_scale: finite; multiplies the renormalised routed weights       */
typedef struct moe_layer_desc {
    int32_t hidden;
    int32_t inter;
    int32_t n_routed;
    int32_t top_k;
    int32_t n_shared;
    int32_t group_size;
    float routed_scale;
} moe_layer_desc;

/* Largest token count one call accepts. */
#define MOE_MAX_TOKENS (1 << 20)

/* ---------------------------------------------------------------------- */
/* Bytes of the caller workspace that moe_permute and moe_route_permute need */
/* at T tokens: a 256-byte header, plus, when T > 1024, 1280 bytes per chunk */
/* of 1024 tokens (each chunk's slot counts per expert group, then its first */
/* row in each group: the permutation's prefix sums, kept in linear space   */
/* instead of recounted by every chunk).  0 when desc or T is invalid.      */
/* Layout (informative): int32 word 0 of the header is moe_route_permute's  */
/* arrival counter for T <= 4; it must be zero before the first call and     */
/* every call leaves it zero.  The rest is rewritten by every call.           */
size_t moe_workspace_bytes(const moe_layer_desc *desc, int32_t T);

/* ---------------------------------------------------------------------- */
/* Routing: logits, sigmoid score, fp32-bias selection, renormalised      */
/* weights.  The pages give only that an FP32 gate bias exists (model     */
/* card, "Component precisions"; "Upstream contributions" records a silent */
/* FP32->BF16 downcast as a bug).  This library's definition:              */
/*   logit[t][e] = sum_h x[t][h] * w_router[e][h], fp32, in a fixed order:  */
/*     64 partial sums, partial l accumulates elements 512j + 8l + u         */
/*     (j ascending, u = 0..7) with fused multiply-add, then pairwise        */
/*     sums of partials l and l^d for d = 32,16,8,4,2,1;                     */
/*   s = 1 / (1 + exp(-logit)) with the library's own fp32 exp (Cody-Waite  */
/*     reduction, degree-7 Taylor polynomial);                              */
/*   key = s + gate_bias[e] (fp32); the k largest keys win, ties to the      */
/*     lower expert index, listed by descending key;                         */
/*   topk_w[t][j] = (s_j / (s_0 + ... + s_{k-1})) * routed_scale, the sum    */
/*     taken in slot order.  The bias only selects.                          */
/* Arguments:                                                                */
/*   x          bf16 [T][H], 16-byte aligned                                 */
/*   w_router   bf16 [E][H], 16-byte aligned                                 */
/*   gate_bias  fp32 [E]                                                     */
/*   logits     fp32 [T][E]   (written; also the input of the selection)     */
/*   topk_idx   int32 [T][k]  (written)                                      */
/*   topk_w     fp32 [T][k]   (written)                                      */
/* Inputs must be finite.                                                    */
moe_status moe_route(const moe_layer_desc *desc, int32_t T, const uint16_t *x,
                     const uint16_t *w_router, const float *gate_bias, float *logits,
                     int32_t *topk_idx, float *topk_w, void *stream);

/* ---------------------------------------------------------------------- */
/* Permutation by expert ("indexed" MoE GEMM rows, "Throughputmaxxing ...",  */
/* "A pass through the model").  The T*(k+n_shared) slots are sorted by     */
/* group with a stable counting sort: slot j<k of token t goes to group     */
/* topk_idx[t][j], slot k (if n_shared) to group E; inside a group rows      */
/* keep the flat slot order t*(k+n_shared)+j.  G = E + n_shared groups,      */
/* R = T*(k+n_shared) rows.                                                  */
/*   topk_idx      int32 [T][k], each row k distinct values in [0,E)         */
/*   group_offsets int32 [G+1]  (written; exclusive prefix sum, [G] = R)     */
/*   sorted_token  int32 [R]    (written; token of each permuted row)        */
/*   row_of_slot   int32 [T][k+n_shared] (written; permuted row of a slot)    */
/*   ws, ws_bytes  workspace of at least moe_workspace_bytes(desc, T) bytes,   */
/*                 16-byte aligned (MOE_ERR_WORKSPACE if smaller, MOE_ERR_NULL */
/*                 if NULL, MOE_ERR_ALIGN if misaligned); used only when     */
/*                 T > 1024 (otherwise it may be NULL)                       */
/* Out-of-range or repeated expert ids give unspecified (but in-bounds)      */
/* results.  Up to 1024 tokens the sort is one launch; past that, three      */
/* (per-chunk counts, their prefix sums, the stable scatter), each linear    */
/* in T.                                                                     */
moe_status moe_permute(const moe_layer_desc *desc, int32_t T, const int32_t *topk_idx,
                       int32_t *group_offsets, int32_t *sorted_token, int32_t *row_of_slot,
                       void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------- */
/* moe_route followed by moe_permute, with the same arguments and results.   */
/* For T <= 4 it is one launch: the router workgroups count themselves on   */
/* the workspace's counter (header word 0) and the last one selects and     */
/* sorts (the decode path); larger T runs the separate kernels.              */
/*   ws, ws_bytes  workspace of at least moe_workspace_bytes(desc, T) bytes,   */
/*                 16-byte aligned, required for every T > 0; zero before     */
/*                 the first call (every call leaves its counter zero).       */
/*                 Calls that may overlap in time (other streams) need        */
/*                 distinct workspaces.                                       */
moe_status moe_route_permute(const moe_layer_desc *desc, int32_t T, const uint16_t *x,
                             const uint16_t *w_router, const float *gate_bias, float *logits,
                             int32_t *topk_idx, float *topk_w, int32_t *group_offsets,
                             int32_t *sorted_token, int32_t *row_of_slot, void *ws,
                             size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------- */
/* moe_route_permute without a workspace argument, for callers that cannot  */
/* allocate device memory: code under HIP graph capture, tight serving      */
/* loops, harnesses that forbid hipMalloc.  The workspace is the library's  */
/* own static device array of MOE_NOALLOC_WS_BYTES bytes, one per GPU, held */
/* until the process ends; the call allocates and frees nothing.  Arguments */
/* and results as moe_route_permute (without ws, ws_bytes).                  */
/*   T            0..MOE_NOALLOC_MAX_TOKENS; larger T returns              */
/*                MOE_ERR_WORKSPACE with nothing enqueued                    */
/* Every call on one GPU shares that GPU's array: calls that may overlap in */
/* time on one GPU (other streams, other threads) race and give unspecified */
/* results.  The first call on a device also enqueues one small kernel that */
/* zeroes the array's counter.  MOE_ERR_DEVICE when no device is current.   */
#define MOE_NOALLOC_MAX_TOKENS 65536
#define MOE_NOALLOC_WS_BYTES 82176
moe_status moe_route_permute_noalloc(const moe_layer_desc *desc, int32_t T, const uint16_t *x,
                                     const uint16_t *w_router, const float *gate_bias,
                                     float *logits, int32_t *topk_idx, float *topk_w,
                                     int32_t *group_offsets, int32_t *sorted_token,
                                     int32_t *row_of_slot, void *stream);

/* ---------------------------------------------------------------------- */
/* Grouped W4A16 GEMM over the permuted rows: for each group g and row r in  */
/* [group_offsets[g], group_offsets[g+1]):                                   */
/*     acc[r][n] = sum_k A[r][k] * q_g[n][k] * s_g[n][k/128]   (fp32)         */
/* then out = bf16(acc) (MOE_ACT_NONE) or bf16(silu(gate)*up) (SWIGLU).      */
/* INT4 codes q are symmetric, zero point 0, in [-8,7]; one fp16 scale per   */
/* 128 consecutive k (model card, "Component precisions": INT4,              */
/* group_size=128, symmetric).                                               */
/*   a            bf16; with a_gather: [n_src][K] and row r reads            */
/*                a[a_gather[r]] (rows outside [0,n_src) read as zero);      */
/*                without: [R][K] and row r reads a[r].  16-byte aligned.    */
/*   n_src        number of rows of a when a_gather is given (>= 1)          */
/*   a_sums       optional (NULL allowed): fp32 [rows of a][K/128], the sum   */
/*                of each row of a over each 128-wide k group, as written by */
/*                moe_row_sums; indexed like a (by a_gather when given).     */
/*                From T >= MOE_TILED_MIN_TOKENS the GEMM uses it for the    */
/*                code-offset correction (-136 x the row sum, see the unpack */
/*                in the kernel) instead of computing it on the matrix       */
/*                cores; below that it is ignored.  Results with and without */
/*                it agree to fp32 rounding.                                  */
/*   N, K         output and input width; N multiple of 64 (<= 65536), K     */
/*                multiple of 128 with K/128 in {1,2,3,4,6,8,12,16,24,32}    */
/*   w_packed     INT4 codes in the kernel layout written by                 */
/*                moe_w4a16_prepack, G*N*K/2 bytes, 16-byte aligned          */
/*   w_scales     fp16 [G][N][K/128] (canonical layout)                      */
/*   group_offsets int32 [G+1] as written by moe_permute                     */
/*   out          bf16 [R][N] (NONE) or [R][N/2] (SWIGLU), 16-byte aligned   */
/* G = E + n_shared and R = T*(k+n_shared) come from desc and T.             */
moe_status moe_w4a16_grouped_gemm(const moe_layer_desc *desc, int32_t T, const uint16_t *a,
                                  const int32_t *a_gather, int32_t n_src, const float *a_sums,
                                  int32_t N, int32_t K, const uint8_t *w_packed,
                                  const uint16_t *w_scales, const int32_t *group_offsets,
                                  int32_t act, uint16_t *out, void *stream);

/* ---------------------------------------------------------------------- */
/* The same grouped GEMM with FP4 expert weights, the format the release     */
/* ships its routed experts in ("Throughputmaxxing: DeepSeek-V4-Flash on     */
/* Isambard-AI", "A pass through the model"; "DeepSeek V4 Flash serving      */
/* hardware", "Released precision").  Element: E2M1 (sign bit 3, exponent    */
/* bits 2..1 with bias 1, mantissa bit 0; values 0, 0.5, 1, 1.5, 2, 3, 4, 6   */
/* and their negatives).  Scale: one UE8M0 byte E per 32 consecutive         */
/* elements along K, meaning 2^(E-127) (E = 255 is not a number; products    */
/* below 2^-126 follow the hardware conversion).  The weights are converted  */
/* to bf16 exactly (two significant bits times a power of two) and the       */
/* products accumulate in fp32 with no per-group rescaling.                  */
/* Arguments as moe_w4a16_grouped_gemm, except:                              */
/*   w_packed     E2M1 codes in the layout written by moe_mxfp4_prepack,     */
/*                G*N*K/2 bytes, 16-byte aligned                              */
/*   w_scales     UE8M0 bytes [G][N][K/32] (canonical layout), 16-byte      */
/*                aligned                                                    */
/*   N, K         N multiple of 128 (<= 65536), K multiple of 128 (<= 4096)  */
/* There is no a_sums argument (no offset term).  Like the INT4 GEMM it runs */
/* the weight-streaming kernel below MOE_TILED_MIN_TOKENS tokens (when K/128 */
/* is one of 1,2,3,4,6,8,12,16,24,32) and the LDS-tiled kernel otherwise.    */
moe_status moe_mxfp4_grouped_gemm(const moe_layer_desc *desc, int32_t T, const uint16_t *a,
                                  const int32_t *a_gather, int32_t n_src, int32_t N, int32_t K,
                                  const uint8_t *w_packed, const uint8_t *w_scales,
                                  const int32_t *group_offsets, int32_t act, uint16_t *out,
                                  void *stream);

/* Token count from which moe_w4a16_grouped_gemm takes its LDS-tiled kernel  */
/* (when N is a multiple of 128 and K <= 4096) and reads a_sums, for both    */
/* projections; below it the weight-streaming kernel (a layer at 256 tokens  */
/* runs 13% faster on it, at 384 both take the same time, at 512 the tiled   */
/* kernel is 11% faster).                                                    */
#define MOE_TILED_MIN_TOKENS 384

/* ---------------------------------------------------------------------- */
/* Row sums over 128-wide k groups, the input a_sums of the GEMM:            */
/*   sums[r][g] = sum_{k in [128g, 128g+128)} a[r][k]   in fp32               */
/* (each lane adds eight consecutive elements in order, then sixteen lanes    */
/* combine pairwise).                                                          */
/*   rows         0..MOE_MAX_TOKENS*9                                         */
/*   K            multiple of 128, <= 65536                                   */
/*   a            bf16 [rows][K], 16-byte aligned                             */
/*   sums         fp32 [rows][K/128] (written)                                */
moe_status moe_row_sums(int32_t rows, int32_t K, const uint16_t *a, float *sums, void *stream);

/* ---------------------------------------------------------------------- */
/* Weighted combine with the shared expert.  Every token's output is its     */
/* six routed experts' outputs weighted by the routing weights plus the one  */
/* always-on shared expert's ("DeepSeek V4 Flash serving hardware", 01,      */
/* "Sparse architecture": one shared expert and six routed experts active   */
/* per token; the shared expert's weight is 1, the routed weights are        */
/* renormalised over the chosen six, this library's reading):                */
/*   out[t] = bf16( y[row_of_slot[t][k]] + sum_j topk_w[t][j] *              */
/*                  y[row_of_slot[t][j]] )  (fp32 sums; shared term only if  */
/*   n_shared, with weight 1).                                               */
/*   y            bf16 [R][H], 16-byte aligned                               */
/*   row_of_slot  int32 [T][k+n_shared] (values in [0,R))                    */
/*   topk_w       fp32 [T][k]                                                */
/*   out          bf16 [T][H], 16-byte aligned                               */
moe_status moe_combine(const moe_layer_desc *desc, int32_t T, const uint16_t *y,
                       const int32_t *row_of_slot, const float *topk_w, uint16_t *out,
                       void *stream);

/* ---------------------------------------------------------------------- */
/* Down projection and weighted combine in one call, for decode batches:     */
/*   out[t] = bf16( y_shared + sum_j topk_w[t][j] * y_j )  with              */
/*   y_j = h[row_of_slot[t][j]] . W2_{g_j}^T,  g_j = topk_idx[t][j] (j < k), */
/*   and the shared expert (group E, weight 1) as slot k when n_shared.     */
/* The same result as moe_w4a16_grouped_gemm(MOE_ACT_NONE) followed by       */
/* moe_combine, except that y is kept in fp32 (not rounded to bf16) and      */
/* never stored.  Each output column block streams the weight rows of every */
/* slot; for T <= MOE_DOWN_COMBINE_MAX_TOKENS only.                          */
/*   h            bf16 [R][I] (the gate/up output), 16-byte aligned          */
/*   w_packed     down codes in the streamed layout, G*H*I/2 bytes           */
/*   w_scales     fp16 [G][H][I/128]                                         */
/*   topk_idx     int32 [T][k], topk_w fp32 [T][k], row_of_slot as written   */
/*                by moe_permute                                             */
/*   out          bf16 [T][H]                                                */
/* Limits: T <= MOE_DOWN_COMBINE_MAX_TOKENS (else MOE_ERR_UNSUPPORTED),      */
/* I/128 in {4, 8, 16, 32} (else MOE_ERR_UNSUPPORTED).                       */
#define MOE_DOWN_COMBINE_MAX_TOKENS 4
moe_status moe_w4a16_down_combine(const moe_layer_desc *desc, int32_t T, const uint16_t *h,
                                  const uint8_t *w_packed, const uint16_t *w_scales,
                                  const int32_t *topk_idx, const float *topk_w,
                                  const int32_t *row_of_slot, uint16_t *out, void *stream);

/* ---------------------------------------------------------------------- */
/* The whole layer for ONE token in one launch (the bs = 1 decode step):    */
/* moe_route_permute, the gate/up GEMM with SwiGLU and moe_w4a16_down_combine */
/* with T = 1, as one persistent kernel of one workgroup per compute unit.  */
/* The selection is bit-identical to moe_route (same definition and code);  */
/* h and out agree with the separate calls to fp32 rounding (the sums are   */
/* associated differently).  What one workgroup needs from the others (the */
/* E scores before the selection, every h tile before the down projection) */
/* passes through `workspace`; a wait that lasts longer than 100 ms (the     */
/* workgroups were not all resident) gives up: it sets word 3 of the        */
/* workspace to 1 and the call's outputs are unspecified.  The raised word  */
/* is sticky: every later call on that workspace returns at once without    */
/* writing its outputs (they stay unspecified) until the caller, after      */
/* synchronising, zeroes the whole workspace again.  Callers check word 3    */
/* after synchronising (the Python binding's Buffers.check_decode does).     */
/* Arguments: as for moe_route_permute (x, w_router, gate_bias and the       */
/* routing outputs, T = 1), the gate/up weights w13_packed/w13_scales        */
/* ([G][2I][H] in the streamed layout, fp16 [G][2I][H/128], both 16-byte     */
/* aligned), the down weights w2_packed/w2_scales ([G][H][I], 16-byte        */
/* aligned, fp16 [G][H][I/128], 4-byte aligned), and                         */
/*   h          bf16 [k+n_shared][I] (written: the gate/up output, in       */
/*              permuted row order), 16-byte aligned                         */
/*   out        bf16 [H] (written), 16-byte aligned                          */
/*   workspace  MOE_DECODE_WORKSPACE_BYTES, 16-byte aligned, all zero before */
/*              the first call and not written by the caller between calls   */
/*              (the calls leave epoch-tagged words in it, never reset); its */
/*              word 3 is raised to 1 by a call that timed out, and word 4   */
/*              counts the calls.  Calls that may overlap in time need       */
/*              distinct workspaces.                                         */
/* Supported shapes (else MOE_ERR_UNSUPPORTED; see                           */
/* moe_w4a16_decode_token_supported): H in {2048, 4096}, (k+n_shared)*I/128  */
/* <= 112, and on the current device at least H/16 compute units, at least  */
/* 2*I/16 when n_shared, at least E/4 and at least k*I/48, and at most 256.  */
/* MOE_ERR_DEVICE when no device is current.                                  */
#define MOE_DECODE_WORKSPACE_BYTES 131072
moe_status moe_w4a16_decode_token(const moe_layer_desc *desc, const uint16_t *x,
                                  const uint16_t *w_router, const float *gate_bias,
                                  const uint8_t *w13_packed, const uint16_t *w13_scales,
                                  const uint8_t *w2_packed, const uint16_t *w2_scales, float *logits,
                                  int32_t *topk_idx, float *topk_w, int32_t *group_offsets,
                                  int32_t *sorted_token, int32_t *row_of_slot, uint16_t *h,
                                  uint16_t *out, int32_t *workspace, void *stream);

/* MOE_OK when moe_w4a16_decode_token supports `desc` on the current device, */
/* else the status that call would return (nothing is enqueued).  The same  */
/* answer holds for moe_mxfp4_decode_token and moe_w4a8_decode_token.        */
moe_status moe_w4a16_decode_token_supported(const moe_layer_desc *desc);

/* The one-launch step with FP4 expert weights (the format of                 */
/* moe_mxfp4_grouped_gemm): w13_packed/w2_packed in the layout written by     */
/* moe_mxfp4_prepack; w13_scales UE8M0 [G][2I][H/32] (16-byte aligned),       */
/* w2_scales UE8M0 [G][H][I/32] (4-byte aligned).  Everything else, the       */
/* workspace included, as moe_w4a16_decode_token.                             */
moe_status moe_mxfp4_decode_token(const moe_layer_desc *desc, const uint16_t *x,
                                  const uint16_t *w_router, const float *gate_bias,
                                  const uint8_t *w13_packed, const uint8_t *w13_scales,
                                  const uint8_t *w2_packed, const uint8_t *w2_scales, float *logits,
                                  int32_t *topk_idx, float *topk_w, int32_t *group_offsets,
                                  int32_t *sorted_token, int32_t *row_of_slot, uint16_t *h,
                                  uint16_t *out, int32_t *workspace, void *stream);

/* ---------------------------------------------------------------------- */
/* fp8 activations.  The pages' faster MoE backend multiplies e4m3          */
/* activations, scaled per token per 128 elements, with 4-bit expert        */
/* weights upcast to fp8 ("Throughputmaxxing: DeepSeek-V4-Flash on          */
/* Isambard-AI", "A pass through the model", W4A8 on fp8 tensor cores); the */
/* attention projections are FP8_BLOCK 128x128 with dynamic ue8m0 scales    */
/* (model card, "Component precisions").  This library's reading of the     */
/* activation format: e4m3 = OCP E4M3FN (largest finite 448); per row and   */
/* per 128 consecutive elements a UE8M0 byte E (scale 2^(E-127)) with       */
/* 2^(E-127) the smallest power of two such that max|x| <= 448 * 2^(E-127)  */
/* (E clamped to [0, 254]; a block of zeros takes E = 127), and each code   */
/* the nearest e4m3 value to x / 2^(E-127), ties to the even code.          */
/*   rows   0..MOE_MAX_TOKENS*9;  K multiple of 128, <= 65536                */
/*   a      bf16 [rows][K], 16-byte aligned                                  */
/*   codes  e4m3 [rows][K] (written), 8-byte aligned                         */
/*   scales UE8M0 [rows][K/128] (written)                                    */
moe_status moe_act_quant_fp8(int32_t rows, int32_t K, const uint16_t *a, uint8_t *codes,
                             uint8_t *scales, void *stream);

/* moe_act_quant_fp8 that also writes each quantised value back in bf16:     */
/*   deq[r][k] = bf16(code[r][k] * 2^(E-127))  (E: its block's scale code)    */
/* -- the value moe_w4a8_grouped_gemm multiplies for that element.  An e4m3  */
/* value has at most four significant bits, so this is exact whenever it is */
/* a multiple of bf16's smallest subnormal, 2^-133: for every nonzero code   */
/* of a block with E >= 3, i.e. a block maximum above 448 * 2^-125; below    */
/* that the value is rounded to the nearest bf16.  A bf16 GEMM on deq then   */
/* multiplies the W4A8 operands exactly (the W4A8 layer does so below        */
/* MOE_TILED_MIN_TOKENS tokens, with the FP4 weight-stream kernels).         */
/*   rows, K, a, codes, scales: as moe_act_quant_fp8                         */
/*   deq    bf16 [rows][K] (written), 16-byte aligned, not overlapping a     */
/*          (MOE_ERR_SHAPE if it does)                                       */
moe_status moe_act_quant_fp8_dequant(int32_t rows, int32_t K, const uint16_t *a, uint8_t *codes,
                                     uint8_t *scales, uint16_t *deq, void *stream);

/* The grouped GEMM of moe_mxfp4_grouped_gemm with fp8 activations (W4A8):   */
/* for each group g and row r of it,                                         */
/*   acc[r][n] = sum_k deq(a)[r][k] * deq(w_g)[n][k]   (fp32)                */
/* deq(a) = e4m3 code times its row's UE8M0 scale of k/128, deq(w) = E2M1    */
/* code times its UE8M0 scale of k/32 -- both scales applied exactly on the  */
/* matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4) -- then out = bf16(acc)  */
/* (MOE_ACT_NONE) or bf16(silu(gate)*up) (MOE_ACT_SWIGLU).                   */
/*   a          e4m3 [n_src][K] (with a_gather) or [R][K], 16-byte aligned   */
/*   a_scales   UE8M0 [n_src or R][K/128], as written by moe_act_quant_fp8  */
/*   a_gather, n_src, group_offsets, act, out: as moe_w4a16_grouped_gemm     */
/*   w_packed, w_scales: as moe_mxfp4_grouped_gemm (the FP4 layout of        */
/*              moe_mxfp4_prepack, UE8M0 [G][N][K/32])                      */
/*   N, K       N multiple of 256 (<= 65536), K multiple of 128 (<= 4096)    */
moe_status moe_w4a8_grouped_gemm(const moe_layer_desc *desc, int32_t T, const uint8_t *a,
                                 const uint8_t *a_scales, const int32_t *a_gather, int32_t n_src,
                                 int32_t N, int32_t K, const uint8_t *w_packed,
                                 const uint8_t *w_scales, const int32_t *group_offsets,
                                 int32_t act, uint16_t *out, void *stream);

/* The W4A8 layer for one token in one launch: moe_mxfp4_decode_token's      */
/* step (the same arguments, layouts, workspace and supported shapes) with   */
/* the expert GEMMs on x and on h quantised as moe_act_quant_fp8 quantises   */
/* them (e4m3 codes with one UE8M0 scale per 128 consecutive elements, "A   */
/* pass through the model" in "Throughputmaxxing: DeepSeek-V4-Flash on       */
/* Isambard-AI"); the router reads x unquantised, as moe_route does.  h is  */
/* written in bf16 before its quantisation, as the W4A8 grouped GEMM writes */
/* it; the quantised codes are not written.  The products of the quantised */
/* values are formed exactly and summed in fp32 in an order of its own, so  */
/* out matches the separate launches (route, quantise, moe_w4a8_grouped_gemm */
/* twice, combine) within rounding, not bit for bit.                         */
moe_status moe_w4a8_decode_token(const moe_layer_desc *desc, const uint16_t *x,
                                 const uint16_t *w_router, const float *gate_bias,
                                 const uint8_t *w13_packed, const uint8_t *w13_scales,
                                 const uint8_t *w2_packed, const uint8_t *w2_scales, float *logits,
                                 int32_t *topk_idx, float *topk_w, int32_t *group_offsets,
                                 int32_t *sorted_token, int32_t *row_of_slot, uint16_t *h,
                                 uint16_t *out, int32_t *workspace, void *stream);

/* FP8_BLOCK GEMM (dense): out[m][n] = bf16( sum_k deq(a)[m][k] *            */
/* deq(w)[n][k] ), deq(w) = e4m3 code times the UE8M0 scale of its 128x128   */
/* block, both scales applied on the matrix cores, fp32 accumulation.        */
/*   M          0..MOE_MAX_TOKENS                                            */
/*   N, K       N multiple of 256 (<= 65536), K multiple of 128 (<= 4096)    */
/*   a, a_scales  e4m3 [M][K] (16-byte aligned) and UE8M0 [M][K/128], as     */
/*              written by moe_act_quant_fp8                                 */
/*   w_packed   e4m3 weights in the layout written by moe_fp8_prepack,       */
/*              N*K bytes, 16-byte aligned                                   */
/*   w_scales   UE8M0 [N/128][K/128]                                         */
/*   out        bf16 [M][N], 4-byte aligned                                  */
moe_status moe_fp8_block_gemm(int32_t M, int32_t N, int32_t K, const uint8_t *a,
                              const uint8_t *a_scales, const uint8_t *w_packed,
                              const uint8_t *w_scales, uint16_t *out, void *stream);

/* Canonical e4m3 weights [N][K] into the layout of moe_fp8_block_gemm: one  */
/* 2048-byte block per (16-row tile nt, 128-wide k group kg) at              */
/* (nt*K/128 + kg)*2048; inside it lane l = (n%16) + 16q owns two 16-byte    */
/* pieces, half h at [1024h + 16l, 1024h + 16l + 16): k = 128kg + 64h + 16q  */
/* + [0,16).                                                                  */
/*   N multiple of 16, K multiple of 128; both buffers N*K bytes, 16-byte    */
/*   aligned, not overlapping                                                */
moe_status moe_fp8_prepack(int32_t N, int32_t K, const uint8_t *w_canonical, uint8_t *w_packed,
                           void *stream);

/* ---------------------------------------------------------------------- */
/* Weight layout.                                                             */
/* Canonical layout (what a checkpoint holds): codes [G][N][K/2] bytes, byte  */
/* c of a row holds element 2c in its low nibble and 2c+1 in its high nibble, */
/* two's complement.  moe_w4a16_prepack rewrites it, bijectively, into the    */
/* layout the GEMM streams: for group g, 16-row tile nt = n/16 and 128-wide   */
/* k group kg, one 1024-byte block at ((g*N/16 + nt)*K/128 + kg)*1024; inside */
/* it lane l = (n%16) + 16*((k%128)/32) owns bytes [16l, 16l+16) = four       */
/* 32-bit words, word d covering k = kg*128 + 32*(l/16) + 8d + [0,8):         */
/* element 2j at bits [4j,4j+4), element 2j+1 at bits [16+4j,20+4j),          */
/* each code stored as (q + 8) (offset binary).                               */
/*   w_canonical  G*N*K/2 bytes, 4-byte aligned                               */
/*   w_packed     G*N*K/2 bytes, 16-byte aligned, must not overlap the input  */
moe_status moe_w4a16_prepack(int32_t n_groups, int32_t N, int32_t K, const uint8_t *w_canonical,
                             uint8_t *w_packed, void *stream);

/* FP4 codes (canonical like the INT4 codes: byte c of a row holds element   */
/* 2c in its low nibble) into the blocks of moe_mxfp4_grouped_gemm: the same */
/* 1024-byte blocks and lane ownership as above, each 32-bit word copied as  */
/* it is (element j of its eight at bits [4j, 4j+4)).  Arguments and limits  */
/* as moe_w4a16_prepack.                                                      */
moe_status moe_mxfp4_prepack(int32_t n_groups, int32_t N, int32_t K, const uint8_t *w_canonical,
                             uint8_t *w_packed, void *stream);

/* ---------------------------------------------------------------------- */
/* Synthetic weight generation on the device (inputs for tests and the       */
/* benchmark; not part of the layer).  Counter-based SplitMix64 (Steele, Lea  */
/* & Flood 2014): output i of the stream seeded with S is                     */
/* mix(S + (i+1)*0x9E3779B97F4A7C15).  Tensor (layer, group, kind) uses       */
/* S = output number ((layer*512 + group)*4 + kind) of the stream seeded with */
/* `seed`.  kind: 0 gate/up codes, 1 down codes, 2 gate/up scales, 3 down     */
/* scales.                                                                    */
/* moe_gen_int4_codes: canonical codes [n_groups][N][K/2] for groups          */
/*   group0.., word i of a tensor = bytes 8i..8i+7 (little endian).           */
/* moe_gen_fp16_scales: fp16 [n_groups][N][K/128]; element i: u = (h>>40)     */
/*   * 2^-24, s = fmaf(0.015, u, 0.005) rounded to fp16.                      */
moe_status moe_gen_int4_codes(uint64_t seed, int32_t layer, int32_t group0, int32_t n_groups,
                              int32_t kind, int32_t N, int32_t K, uint8_t *out, void *stream);
moe_status moe_gen_fp16_scales(uint64_t seed, int32_t layer, int32_t group0, int32_t n_groups,
                               int32_t kind, int32_t N, int32_t K, uint16_t *out, void *stream);
/* moe_gen_ue8m0_scales: UE8M0 bytes [n_groups][N][K/32] (K multiple of 32);  */
/*   element i: E = 120 + (h >> 62).  FP4 codes come from moe_gen_int4_codes  */
/*   (the same uniform nibbles).                                              */
moe_status moe_gen_ue8m0_scales(uint64_t seed, int32_t layer, int32_t group0, int32_t n_groups,
                                int32_t kind, int32_t N, int32_t K, uint8_t *out, void *stream);

/* Human-readable name of a status (static string, never NULL). */
const char *moe_status_str(moe_status status);

/* ABI version of this header (bumped on any incompatible change). */
#define MOE_W4A16_ABI_VERSION 10
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4A16_H */
