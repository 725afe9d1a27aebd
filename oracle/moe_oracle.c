/*
 * moe_oracle.c -- plain, slow CPU oracle of the W4A16 routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or constant with the HIP library; every constant below is
 * derived here from its definition.
 *
 * What the layer computes (DeepSeek-V4-Flash MoE layer as described on the
 * pages):
 *   - 256 routed experts with 6 active per token plus one always-on shared
 *     expert, hidden size 4096 ("DeepSeek V4 Flash serving hardware", 01
 *     source-pinned baseline, "Sparse architecture"; model card
 *     "canada-quant/DeepSeek-V4-Flash-W4A16-FP8-MTP", "Architecture & precision",
 *     base-model table);
 *   - routed experts hold three projections in W4A16 INT4, group_size=128,
 *     symmetric (model card, "Component precisions" table);
 *   - ffn.gate.bias is FP32 (same table, and "Upstream contributions");
 *   - the layer is weight-only: 4-bit weights are dequantised to 16-bit and
 *     multiplied with 16-bit activations ("Throughputmaxxing: DeepSeek-V4-Flash on
 *     Isambard-AI", section "A pass through the model", on Marlin).
 * The same layer with FP4 expert weights (the format the release ships)
 * differs only in how a weight is dequantised (oracle_dequant_fp4_rows).
 * The pages give no router formula, activation, nibble order or scale dtype;
 * the readings taken for those are stated next to each function.
 *
 * Precision: routing is computed in fp32 in a fully specified order (it
 * decides integers: the chosen experts), the expert MLPs and the combine in
 * fp64.  Activations handed from one step to the next (h, y, out) are rounded
 * to bf16 -- the "A16" of W4A16.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#pragma STDC FP_CONTRACT OFF

/* ------------------------------------------------------------------ */
/* storage formats                                                     */
/* ------------------------------------------------------------------ */
static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* IEEE binary16 -> double, written from the format definition. */
double oracle_fp16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);              /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25); /* (1024+m) * 2^(e-15-10) */
    return sign ? -v : v;
}

/* double -> bf16, round to nearest, ties to even, in one rounding step. */
uint16_t oracle_f64_to_bf16(double x)
{
    if (isnan(x)) return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    double q;
    if (a < ldexp(1.0, -126)) {
        q = nearbyint(ldexp(a, 133));            /* subnormal grid: 2^-133 */
        a = ldexp(q, -133);
    } else {
        int e;
        double m = frexp(a, &e);                 /* a = m * 2^e, m in [0.5,1) */
        q = nearbyint(ldexp(m, 8));              /* 8 significant bits */
        a = ldexp(q, e - 8);
    }
    if (a >= ldexp(1.0, 128)) return sign | 0x7F80; /* overflow -> inf */
    float f = (float)a;                          /* exact: a has <= 8 bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return sign | (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------ */
/* O1 dequantisation                                                   */
/* Reading: two's-complement codes in [-8,7], zero point 0; byte c of a  */
/* row holds element 2c in its low nibble and 2c+1 in its high nibble;   */
/* one fp16 scale per 128 consecutive elements along K (model card,      */
/* "Component precisions": INT4, group_size=128, symmetric).            */
/* ------------------------------------------------------------------ */
int oracle_int4_code(uint8_t byte, int high)
{
    int nib = high ? (byte >> 4) : (byte & 0xF);
    return nib >= 8 ? nib - 16 : nib;
}

/* Dequantised weight (n, k) of a canonical [N][K/2] code array with
 * [N][K/128] fp16 scales.  q*s has <= 15 significant bits: exact in double. */
static double deq(const uint8_t *w, const uint16_t *s, int K, int n, int k)
{
    uint8_t byte = w[(size_t)n * (K / 2) + (k >> 1)];
    int q = oracle_int4_code(byte, k & 1);
    return (double)q * oracle_fp16_to_f64(s[(size_t)n * (K / 128) + (k >> 7)]);
}

void oracle_dequant_rows(int N, int K, const uint8_t *w, const uint16_t *s, double *out)
{
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            out[(size_t)n * K + k] = deq(w, s, K, n, k);
}

/* ------------------------------------------------------------------ */
/* FP4 expert weights.  The release's routed experts ship in fp4       */
/* ("Throughputmaxxing: DeepSeek-V4-Flash on Isambard-AI", "A pass     */
/* through the model"; "DeepSeek V4 Flash serving hardware", "Released */
/* precision").  The pages give no element or scale format; reading:   */
/* the OCP microscaling FP4 element E2M1 (sign bit 3, exponent bits    */
/* 2..1 with bias 1, mantissa bit 0; exponent 0 holds 0 and 0.5) with  */
/* one power-of-two scale UE8M0 = 2^(E-127) (E = 255: not a number)    */
/* per 32 consecutive elements along K.  Codes pack like the INT4      */
/* codes: byte c of a row holds element 2c in its low nibble.          */
/* ------------------------------------------------------------------ */
double oracle_fp4_value(int code)
{
    int sign = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -v : v;
}

double oracle_ue8m0(int E)
{
    return E == 255 ? NAN : ldexp(1.0, E - 127);
}

/* an E2M1 value (2 significant bits) times a power of two: exact */
static double deq_fp4(const uint8_t *w, const uint8_t *s, int K, int n, int k)
{
    uint8_t byte = w[(size_t)n * (K / 2) + (k >> 1)];
    int code = (k & 1) ? (byte >> 4) : (byte & 0xF);
    return oracle_fp4_value(code) * oracle_ue8m0(s[(size_t)n * (K / 32) + (k >> 5)]);
}

void oracle_dequant_fp4_rows(int N, int K, const uint8_t *w, const uint8_t *s, double *out)
{
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            out[(size_t)n * K + k] = deq_fp4(w, s, K, n, k);
}

/* ------------------------------------------------------------------ */
/* O3 exp and sigmoid (fp32).                                          */
/* Written from the mathematics: Cody & Waite additive range reduction  */
/* y = n ln2 + r with ln2 split in a 12-significant-bit head and a tail, */
/* |r| <= ln2/2, then the degree-7 Taylor polynomial of e^r in Horner   */
/* form with fused multiply-adds, then scaling by 2^n.  Truncation error */
/* r^8/8! <= 5.2e-9, below half an fp32 ulp of e^r.                    */
/* ------------------------------------------------------------------ */
static float f32_from_bits(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    return f;
}

float oracle_exp(float y)
{
    const double LN2 = 0.693147180559945309417232121458;
    const float log2e = (float)(1.0 / LN2);
    /* head: ln2 rounded to fp32, low 12 stored mantissa bits cleared, so
       n * ln2_hi is exact for |n| <= 2^11 */
    uint32_t ln2_bits;
    float ln2f = (float)LN2;
    memcpy(&ln2_bits, &ln2f, 4);
    const float ln2_hi = f32_from_bits(ln2_bits & 0xFFFFF000u);
    const float ln2_lo = (float)(LN2 - (double)ln2_hi);
    const float c2 = (float)(1.0 / 2.0), c3 = (float)(1.0 / 6.0), c4 = (float)(1.0 / 24.0);
    const float c5 = (float)(1.0 / 120.0), c6 = (float)(1.0 / 720.0), c7 = (float)(1.0 / 5040.0);

    if (y >= 88.5f) return INFINITY;
    if (y <= -86.0f) return 0.0f;
    float n = rintf(y * log2e);
    float r = fmaf(-n, ln2_hi, y);
    r = fmaf(-n, ln2_lo, r);
    float p = c7;
    p = fmaf(p, r, c6);
    p = fmaf(p, r, c5);
    p = fmaf(p, r, c4);
    p = fmaf(p, r, c3);
    p = fmaf(p, r, c2);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return ldexpf(p, (int)n);
}

/* Reading (pages silent on the scoring function): sigmoid scores. */
float oracle_sigmoid(float l)
{
    float e = oracle_exp(-l);
    float d = 1.0f + e;
    return 1.0f / d;
}

void oracle_exp_array(int64_t n, const float *y, float *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_exp(y[i]);
}

void oracle_sigmoid_array(int64_t n, const float *y, float *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_sigmoid(y[i]);
}

/* ------------------------------------------------------------------ */
/* O2 router logits, fp32, order fixed so that a 64-lane GPU wavefront  */
/* can reproduce it bit for bit (the expert choice is an integer        */
/* decided by floating point, so both sides decide it in the same       */
/* arithmetic):                                                         */
/*   partial P[l], l in [0,64), starts at +0;                           */
/*   for j in [0, H/512), u in [0,8): i = 512 j + 8 l + u,              */
/*       P[l] = fmaf(x[i], w[i], P[l]);                                 */
/*   then for d = 32,16,8,4,2,1: P[l] = P[l] + P[l xor d] (all l);      */
/*   the logit is P[0].                                                 */
/* ------------------------------------------------------------------ */
static float router_dot(int H, const uint16_t *x, const uint16_t *w)
{
    float P[64], Q[64];
    for (int l = 0; l < 64; ++l) P[l] = 0.0f;
    for (int j = 0; j < H / 512; ++j)
        for (int l = 0; l < 64; ++l)
            for (int u = 0; u < 8; ++u) {
                int i = 512 * j + 8 * l + u;
                P[l] = fmaf(bf16_to_f32(x[i]), bf16_to_f32(w[i]), P[l]);
            }
    for (int d = 32; d >= 1; d >>= 1) {
        for (int l = 0; l < 64; ++l) Q[l] = P[l] + P[l ^ d];
        for (int l = 0; l < 64; ++l) P[l] = Q[l];
    }
    return P[0];
}

void oracle_router_logits(int T, int H, int E, const uint16_t *x, const uint16_t *wr, float *logits)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e)
            logits[(size_t)t * E + e] = router_dot(H, x + (size_t)t * H, wr + (size_t)e * H);
}

/* ------------------------------------------------------------------ */
/* O4 selection.  Reading (pages: only that an fp32 gate bias exists):  */
/*   s_e = sigmoid(logit_e); key_e = s_e + b_e (fp32);                  */
/*   the k chosen experts are the k largest keys, ties to the lower     */
/*   expert index, listed in that order (slot 0 = largest key);         */
/*   weights use the unbiased scores: S = s_e0 + s_e1 + ... (fp32, slot  */
/*   order), w_j = (s_ej / S) * routed_scale.                            */
/* Returns 0, or -1 if a key is not finite.                             */
/* ------------------------------------------------------------------ */
int oracle_select(int T, int E, int k, float routed_scale, const float *logits,
                  const float *bias, int32_t *idx, float *w)
{
    int bad = 0;
    float *s = (float *)malloc(sizeof(float) * E);
    float *key = (float *)malloc(sizeof(float) * E);
    char *taken = (char *)malloc(E);
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            s[e] = oracle_sigmoid(logits[(size_t)t * E + e]);
            key[e] = s[e] + bias[e];
            if (!isfinite(key[e])) bad = 1;
            taken[e] = 0;
        }
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || key[e] > key[best]) best = e; /* ascending e: ties keep lower */
            }
            taken[best] = 1;
            idx[(size_t)t * k + j] = best;
        }
        float S = s[idx[(size_t)t * k]];
        for (int j = 1; j < k; ++j) S = S + s[idx[(size_t)t * k + j]];
        for (int j = 0; j < k; ++j) {
            float q = s[idx[(size_t)t * k + j]] / S;
            w[(size_t)t * k + j] = q * routed_scale;
        }
    }
    free(s);
    free(key);
    free(taken);
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------ */
/* O6 permutation: stable counting sort of the T*(k+ns) slots by group.  */
/* Slot j<k of token t goes to group idx[t][j]; slot k (when ns=1) goes  */
/* to the shared expert, group E.  Within a group rows keep flat slot    */
/* order f = t*(k+ns) + j.  Reading: dropless (no capacity limit).       */
/* ------------------------------------------------------------------ */
int oracle_permute(int T, int E, int k, int ns, const int32_t *idx, int32_t *offsets,
                   int32_t *sorted_token, int32_t *row_of_slot)
{
    int G = E + ns, S = k + ns;
    int64_t *cursor = (int64_t *)calloc((size_t)G + 1, sizeof(int64_t));
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < S; ++j) {
            int g = j < k ? idx[(size_t)t * k + j] : E;
            if (j < k && (g < 0 || g >= E)) { free(cursor); return -1; }
            cursor[g + 1]++;
        }
    for (int g = 0; g < G; ++g) cursor[g + 1] += cursor[g];
    for (int g = 0; g <= G; ++g) offsets[g] = (int32_t)cursor[g];
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < S; ++j) {
            int g = j < k ? idx[(size_t)t * k + j] : E;
            int64_t pos = cursor[g]++;
            sorted_token[pos] = t;
            row_of_slot[(size_t)t * S + j] = (int32_t)pos;
        }
    free(cursor);
    return 0;
}

/* ------------------------------------------------------------------ */
/* O7 expert MLP for n rows through one group (fp64).                   */
/* Reading (pages silent on the activation): SwiGLU.  W13 rows [0,I)    */
/* are the gate projection, rows [I,2I) the up projection:              */
/*   G_n = sum_h x_h w1(n,h),  U_n = sum_h x_h w3(n,h),                 */
/*   h_n = bf16( G_n / (1 + exp(-G_n)) * U_n ),                         */
/*   y_m = bf16( sum_n h_n w2(m,n) ).                                   */
/* Weights are dequantised on the fly from the canonical codes.         */
/* ------------------------------------------------------------------ */
static void mlp_rows(int nrows, int H, int I, const uint16_t *x, const double *w13d,
                     const double *w2d, uint16_t *h_out, uint16_t *y_out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; ++r) {
        const uint16_t *xr = x + (size_t)r * H;
        double *hv = (double *)malloc(sizeof(double) * I);
        for (int n = 0; n < I; ++n) {
            double g = 0.0, u = 0.0;
            const double *wg = w13d + (size_t)n * H, *wu = w13d + (size_t)(I + n) * H;
            for (int h = 0; h < H; ++h) {
                double xv = (double)bf16_to_f32(xr[h]);
                g += xv * wg[h];
                u += xv * wu[h];
            }
            double a = g / (1.0 + exp(-g)) * u;
            uint16_t hb = oracle_f64_to_bf16(a);
            h_out[(size_t)r * I + n] = hb;
            hv[n] = (double)bf16_to_f32(hb);
        }
        for (int m = 0; m < H; ++m) {
            double acc = 0.0;
            const double *wm = w2d + (size_t)m * I;
            for (int n = 0; n < I; ++n) acc += hv[n] * wm[n];
            y_out[(size_t)r * H + m] = oracle_f64_to_bf16(acc);
        }
        free(hv);
    }
}

void oracle_expert_mlp(int nrows, int H, int I, const uint16_t *x, const uint8_t *w13,
                       const uint16_t *s13, const uint8_t *w2, const uint16_t *s2,
                       uint16_t *h_out, uint16_t *y_out)
{
    double *w13d = (double *)malloc(sizeof(double) * (size_t)2 * I * H);
    double *w2d = (double *)malloc(sizeof(double) * (size_t)H * I);
    oracle_dequant_rows(2 * I, H, w13, s13, w13d);
    oracle_dequant_rows(H, I, w2, s2, w2d);
    mlp_rows(nrows, H, I, x, w13d, w2d, h_out, y_out);
    free(w13d);
    free(w2d);
}

/* The same MLP with FP4 weights: scales s13 [2I][H/32], s2 [H][I/32]. */
void oracle_expert_mlp_fp4(int nrows, int H, int I, const uint16_t *x, const uint8_t *w13,
                           const uint8_t *s13, const uint8_t *w2, const uint8_t *s2,
                           uint16_t *h_out, uint16_t *y_out)
{
    double *w13d = (double *)malloc(sizeof(double) * (size_t)2 * I * H);
    double *w2d = (double *)malloc(sizeof(double) * (size_t)H * I);
    oracle_dequant_fp4_rows(2 * I, H, w13, s13, w13d);
    oracle_dequant_fp4_rows(H, I, w2, s2, w2d);
    mlp_rows(nrows, H, I, x, w13d, w2d, h_out, y_out);
    free(w13d);
    free(w2d);
}

/* ------------------------------------------------------------------ */
/* O8 combine: out[t] = bf16( y[shared row] + sum_j w_j * y[row(t,j)] ),  */
/* summed in fp64 (shared expert weight 1, not renormalised).            */
/* ------------------------------------------------------------------ */
void oracle_combine(int T, int H, int k, int ns, const uint16_t *y, const int32_t *row_of_slot,
                    const float *w, uint16_t *out)
{
    int S = k + ns;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int m = 0; m < H; ++m) {
            double acc = 0.0;
            if (ns) acc = (double)bf16_to_f32(y[(size_t)row_of_slot[(size_t)t * S + k] * H + m]);
            for (int j = 0; j < k; ++j)
                acc += (double)w[(size_t)t * k + j] *
                       (double)bf16_to_f32(y[(size_t)row_of_slot[(size_t)t * S + j] * H + m]);
            out[(size_t)t * H + m] = oracle_f64_to_bf16(acc);
        }
}

/* ------------------------------------------------------------------ */
/* The whole layer for small shapes: route, select, permute, every     */
/* group's MLP over its rows, combine.  Canonical weights of all G      */
/* groups are stacked: w13 [G][2I][H/2], s13 [G][2I][H/128],            */
/* w2 [G][H][I/2], s2 [G][H][I/128].  h [R][I], y [R][H] in permuted    */
/* row order.  Returns 0 on success.                                    */
/* ------------------------------------------------------------------ */
int oracle_layer_forward(int T, int H, int I, int E, int k, int ns, float routed_scale,
                         const uint16_t *x, const uint16_t *wr, const float *bias,
                         const uint8_t *w13, const uint16_t *s13, const uint8_t *w2,
                         const uint16_t *s2, float *logits, int32_t *idx, float *w,
                         int32_t *offsets, int32_t *sorted_token, int32_t *row_of_slot,
                         uint16_t *h, uint16_t *y, uint16_t *out)
{
    int G = E + ns;
    oracle_router_logits(T, H, E, x, wr, logits);
    if (oracle_select(T, E, k, routed_scale, logits, bias, idx, w)) return -1;
    if (oracle_permute(T, E, k, ns, idx, offsets, sorted_token, row_of_slot)) return -2;
    for (int g = 0; g < G; ++g) {
        int r0 = offsets[g], n = offsets[g + 1] - offsets[g];
        if (n == 0) continue;
        uint16_t *xg = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)n * H);
        for (int r = 0; r < n; ++r)
            memcpy(xg + (size_t)r * H, x + (size_t)sorted_token[r0 + r] * H, sizeof(uint16_t) * H);
        oracle_expert_mlp(n, H, I, xg, w13 + (size_t)g * 2 * I * (H / 2),
                          s13 + (size_t)g * 2 * I * (H / 128), w2 + (size_t)g * H * (I / 2),
                          s2 + (size_t)g * H * (I / 128), h + (size_t)r0 * I, y + (size_t)r0 * H);
        free(xg);
    }
    oracle_combine(T, H, k, ns, y, row_of_slot, w, out);
    return 0;
}

/* The whole layer with FP4 expert weights: s13 [G][2I][H/32] and
 * s2 [G][H][I/32] UE8M0 bytes; everything else as oracle_layer_forward. */
int oracle_layer_forward_fp4(int T, int H, int I, int E, int k, int ns, float routed_scale,
                             const uint16_t *x, const uint16_t *wr, const float *bias,
                             const uint8_t *w13, const uint8_t *s13, const uint8_t *w2,
                             const uint8_t *s2, float *logits, int32_t *idx, float *w,
                             int32_t *offsets, int32_t *sorted_token, int32_t *row_of_slot,
                             uint16_t *h, uint16_t *y, uint16_t *out)
{
    int G = E + ns;
    oracle_router_logits(T, H, E, x, wr, logits);
    if (oracle_select(T, E, k, routed_scale, logits, bias, idx, w)) return -1;
    if (oracle_permute(T, E, k, ns, idx, offsets, sorted_token, row_of_slot)) return -2;
    for (int g = 0; g < G; ++g) {
        int r0 = offsets[g], n = offsets[g + 1] - offsets[g];
        if (n == 0) continue;
        uint16_t *xg = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)n * H);
        for (int r = 0; r < n; ++r)
            memcpy(xg + (size_t)r * H, x + (size_t)sorted_token[r0 + r] * H, sizeof(uint16_t) * H);
        oracle_expert_mlp_fp4(n, H, I, xg, w13 + (size_t)g * 2 * I * (H / 2),
                              s13 + (size_t)g * 2 * I * (H / 32), w2 + (size_t)g * H * (I / 2),
                              s2 + (size_t)g * H * (I / 32), h + (size_t)r0 * I, y + (size_t)r0 * H);
        free(xg);
    }
    oracle_combine(T, H, k, ns, y, row_of_slot, w, out);
    return 0;
}

/* ------------------------------------------------------------------ */
/* FP8 activations: the W4A8 variant of the layer and the FP8_BLOCK    */
/* projection GEMM.                                                    */
/*                                                                     */
/* The pages: the faster MoE backend upcasts the 4-bit weights to fp8   */
/* and multiplies fp8 x fp8, with the activations in e4m3 scaled per    */
/* token per 128 elements and the per-128 input scales applied on the   */
/* accumulator ("Throughputmaxxing: DeepSeek-V4-Flash on Isambard-AI",  */
/* "A pass through the model": the DeepSeek recipe of 1x128 activation  */
/* tiles); the attention projections are FP8_BLOCK 128x128 with dynamic */
/* scales in scale_fmt=ue8m0 (model card, "Component precisions").      */
/* Readings: e4m3 is the OCP format E4M3FN (bias 7, no infinities, NaN  */
/* only S.1111.111, largest finite 448); an activation scale is the     */
/* smallest power of two 2^e with max|x| <= 448 * 2^e over the block    */
/* (stored as the UE8M0 byte e + 127; a block of zeros takes e = 0),    */
/* and each element is x / 2^e rounded to the nearest e4m3 value, ties  */
/* to the even code.  The weights of the W4A8 variant are the FP4       */
/* expert weights above (E2M1 times their UE8M0 scale: exact in fp64);  */
/* FP8_BLOCK weights are e4m3 codes with one UE8M0 scale per 128x128    */
/* block.  Products and sums in fp64; h between the two GEMMs is stored */
/* as bf16 (as in W4A16) and then quantised like x.                     */
/* ------------------------------------------------------------------ */
double oracle_e4m3_value(int code)
{
    int s = (code >> 7) & 1, e = (code >> 3) & 0xF, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    v = e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10); /* m/8 * 2^-6, (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* Nearest e4m3 value, ties to the even code; |v| >= 448 gives +-448;   */
/* a NaN gives the format's NaN pattern S.1111.111 (E4M3 has no inf).   */
int oracle_e4m3_encode(double v)
{
    int sign = signbit(v) ? 0x80 : 0, e2, m;
    double a = fabs(v), q, n;
    if (isnan(v)) return sign | 0x7F;
    if (a >= 448.0) return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {
        q = ldexp(1.0, -9); /* subnormal spacing */
    } else {
        frexp(a, &e2); /* a = f 2^e2, f in [0.5, 1): a's binade is 2^(e2-1) */
        q = ldexp(1.0, e2 - 1 - 3);
    }
    n = rint(a / q); /* a / q is exact; rint rounds half to even */
    a = n * q;
    if (a == 0.0) return sign;
    if (a < ldexp(1.0, -6)) return sign | (int)(a / ldexp(1.0, -9));
    frexp(a, &e2);
    m = (int)(ldexp(a, -(e2 - 1)) * 8.0) - 8; /* a = (1 + m/8) 2^(e2-1) */
    return sign | ((e2 - 1 + 7) << 3) | m;
}

/* UE8M0 code of the activation scale of n values: the smallest e with  */
/* max|x| <= 448 * 2^e (comparisons exact in fp64), e + 127, clamped to  */
/* [0, 254]; a block of zeros gives 127 (scale 1).                       */
int oracle_act_scale_code(const uint16_t *x, int n)
{
    double amax = 0.0;
    int e;
    for (int i = 0; i < n; ++i) amax = fmax(amax, fabs((double)bf16_to_f32(x[i])));
    if (amax == 0.0) return 127;
    frexp(amax / 448.0, &e);
    while (amax > ldexp(448.0, e)) ++e;
    while (e > -127 && amax <= ldexp(448.0, e - 1)) --e;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e + 127;
}

/* codes [rows][K] (e4m3), scales [rows][K/128] (UE8M0) */
void oracle_act_quant_fp8(int rows, int K, const uint16_t *x, uint8_t *codes, uint8_t *scales)
{
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r)
        for (int b = 0; b < K / 128; ++b) {
            const uint16_t *xb = x + (size_t)r * K + 128 * b;
            int E = oracle_act_scale_code(xb, 128);
            scales[(size_t)r * (K / 128) + b] = (uint8_t)E;
            for (int i = 0; i < 128; ++i)
                codes[(size_t)r * K + 128 * b + i] =
                    (uint8_t)oracle_e4m3_encode(ldexp((double)bf16_to_f32(xb[i]), 127 - E));
        }
}

/* dequantised row of an fp8 activation: codes [K], scales [K/128] */
static void act_dequant_row(int K, const uint8_t *codes, const uint8_t *scales, double *out)
{
    for (int k = 0; k < K; ++k) out[k] = ldexp(oracle_e4m3_value(codes[k]), scales[k / 128] - 127);
}

/* W4A8 expert MLP over nrows rows with FP4 weights (layout of            */
/* oracle_expert_mlp_fp4): x quantised per 128; G, U, silu(G)*U in fp64; */
/* h = bf16 (h_out); h quantised per 128 (hq_codes [n][I], hq_scales     */
/* [n][I/128]); y = bf16(dequantised h . w2).                            */
void oracle_expert_mlp_w4a8(int nrows, int H, int I, const uint16_t *x, const uint8_t *w13,
                            const uint8_t *s13, const uint8_t *w2, const uint8_t *s2,
                            uint16_t *h_out, uint8_t *hq_codes, uint8_t *hq_scales, uint16_t *y_out)
{
    double *w13d = (double *)malloc(sizeof(double) * (size_t)2 * I * H);
    double *w2d = (double *)malloc(sizeof(double) * (size_t)H * I);
    oracle_dequant_fp4_rows(2 * I, H, w13, s13, w13d);
    oracle_dequant_fp4_rows(H, I, w2, s2, w2d);
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; ++r) {
        uint8_t *xc = (uint8_t *)malloc((size_t)H);
        uint8_t *xs = (uint8_t *)malloc((size_t)H / 128);
        double *xd = (double *)malloc(sizeof(double) * H);
        double *hd = (double *)malloc(sizeof(double) * I);
        uint16_t *hr = h_out + (size_t)r * I;
        oracle_act_quant_fp8(1, H, x + (size_t)r * H, xc, xs);
        act_dequant_row(H, xc, xs, xd);
        for (int n = 0; n < I; ++n) {
            double g = 0.0, u = 0.0;
            const double *wg = w13d + (size_t)n * H, *wu = w13d + (size_t)(I + n) * H;
            for (int k = 0; k < H; ++k) {
                g += xd[k] * wg[k];
                u += xd[k] * wu[k];
            }
            hr[n] = oracle_f64_to_bf16(g / (1.0 + exp(-g)) * u);
        }
        oracle_act_quant_fp8(1, I, hr, hq_codes + (size_t)r * I, hq_scales + (size_t)r * (I / 128));
        act_dequant_row(I, hq_codes + (size_t)r * I, hq_scales + (size_t)r * (I / 128), hd);
        for (int m = 0; m < H; ++m) {
            double acc = 0.0;
            const double *wm = w2d + (size_t)m * I;
            for (int n = 0; n < I; ++n) acc += hd[n] * wm[n];
            y_out[(size_t)r * H + m] = oracle_f64_to_bf16(acc);
        }
        free(xc);
        free(xs);
        free(xd);
        free(hd);
    }
    free(w13d);
    free(w2d);
}

/* The whole W4A8 layer (FP4 expert weights as oracle_layer_forward_fp4);
 * h [R][I] bf16, hq codes [R][I] and scales [R][I/128], y [R][H] in
 * permuted row order. */
int oracle_layer_forward_w4a8(int T, int H, int I, int E, int k, int ns, float routed_scale,
                              const uint16_t *x, const uint16_t *wr, const float *bias,
                              const uint8_t *w13, const uint8_t *s13, const uint8_t *w2,
                              const uint8_t *s2, float *logits, int32_t *idx, float *w,
                              int32_t *offsets, int32_t *sorted_token, int32_t *row_of_slot,
                              uint16_t *h, uint8_t *hq_codes, uint8_t *hq_scales, uint16_t *y,
                              uint16_t *out)
{
    int G = E + ns;
    oracle_router_logits(T, H, E, x, wr, logits);
    if (oracle_select(T, E, k, routed_scale, logits, bias, idx, w)) return -1;
    if (oracle_permute(T, E, k, ns, idx, offsets, sorted_token, row_of_slot)) return -2;
    for (int g = 0; g < G; ++g) {
        int r0 = offsets[g], n = offsets[g + 1] - offsets[g];
        if (n == 0) continue;
        uint16_t *xg = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)n * H);
        for (int r = 0; r < n; ++r)
            memcpy(xg + (size_t)r * H, x + (size_t)sorted_token[r0 + r] * H, sizeof(uint16_t) * H);
        oracle_expert_mlp_w4a8(n, H, I, xg, w13 + (size_t)g * 2 * I * (H / 2),
                               s13 + (size_t)g * 2 * I * (H / 32), w2 + (size_t)g * H * (I / 2),
                               s2 + (size_t)g * H * (I / 32), h + (size_t)r0 * I,
                               hq_codes + (size_t)r0 * I, hq_scales + (size_t)r0 * (I / 128),
                               y + (size_t)r0 * H);
        free(xg);
    }
    oracle_combine(T, H, k, ns, y, row_of_slot, w, out);
    return 0;
}

/* FP8_BLOCK GEMM: y [M][N] = bf16( quant(x) . W^T ), x bf16 [M][K],      */
/* W e4m3 codes [N][K] with UE8M0 scales ws [N/128][K/128].               */
void oracle_fp8_block_gemm(int M, int N, int K, const uint16_t *x, const uint8_t *w, const uint8_t *ws,
                           uint16_t *y)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int m = 0; m < M; ++m) {
        uint8_t *xc = (uint8_t *)malloc((size_t)K);
        uint8_t *xs = (uint8_t *)malloc((size_t)K / 128);
        double *xd = (double *)malloc(sizeof(double) * K);
        oracle_act_quant_fp8(1, K, x + (size_t)m * K, xc, xs);
        act_dequant_row(K, xc, xs, xd);
        for (int n = 0; n < N; ++n) {
            double acc = 0.0;
            const uint8_t *wn = w + (size_t)n * K;
            for (int k = 0; k < K; ++k)
                acc += xd[k] * ldexp(oracle_e4m3_value(wn[k]),
                                     ws[(size_t)(n / 128) * (K / 128) + k / 128] - 127);
            y[(size_t)m * N + n] = oracle_f64_to_bf16(acc);
        }
        free(xc);
        free(xs);
        free(xd);
    }
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
