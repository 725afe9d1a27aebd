/* sanitize_main.c -- TEST INFRASTRUCTURE: a driver that runs every function
 * of moe_oracle.c once on small shapes, for an AddressSanitizer /
 * UndefinedBehaviorSanitizer build (tests/test_sanitizers.py).  Every buffer
 * is allocated at exactly the size the function's contract states, so an
 * access one element past it is reported.  The inputs are arbitrary
 * (xorshift); parity is checked elsewhere -- this checks memory safety and
 * defined behaviour only.  Exit status 0 on a clean run. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_fp16_to_f64(uint16_t h);
uint16_t oracle_f64_to_bf16(double x);
int oracle_int4_code(uint8_t byte, int high);
void oracle_dequant_rows(int N, int K, const uint8_t *w, const uint16_t *s, double *out);
double oracle_fp4_value(int code);
double oracle_ue8m0(int E);
void oracle_dequant_fp4_rows(int N, int K, const uint8_t *w, const uint8_t *s, double *out);
float oracle_exp(float y);
float oracle_sigmoid(float l);
void oracle_exp_array(int64_t n, const float *y, float *out);
void oracle_sigmoid_array(int64_t n, const float *y, float *out);
void oracle_router_logits(int T, int H, int E, const uint16_t *x, const uint16_t *wr, float *logits);
int oracle_select(int T, int E, int k, float routed_scale, const float *logits, const float *bias, int32_t *idx,
                  float *w);
int oracle_permute(int T, int E, int k, int ns, const int32_t *idx, int32_t *offsets, int32_t *sorted_token,
                   int32_t *row_of_slot);
void oracle_expert_mlp(int nrows, int H, int I, const uint16_t *x, const uint8_t *w13, const uint16_t *s13,
                       const uint8_t *w2, const uint16_t *s2, uint16_t *h_out, uint16_t *y_out);
void oracle_expert_mlp_fp4(int nrows, int H, int I, const uint16_t *x, const uint8_t *w13, const uint8_t *s13,
                           const uint8_t *w2, const uint8_t *s2, uint16_t *h_out, uint16_t *y_out);
void oracle_combine(int T, int H, int k, int ns, const uint16_t *y, const int32_t *row_of_slot, const float *w,
                    uint16_t *out);
int oracle_layer_forward(int T, int H, int I, int E, int k, int ns, float routed_scale, const uint16_t *x,
                         const uint16_t *wr, const float *bias, const uint8_t *w13, const uint16_t *s13,
                         const uint8_t *w2, const uint16_t *s2, float *logits, int32_t *idx, float *w,
                         int32_t *offsets, int32_t *sorted_token, int32_t *row_of_slot, uint16_t *h, uint16_t *y,
                         uint16_t *out);
int oracle_layer_forward_fp4(int T, int H, int I, int E, int k, int ns, float routed_scale, const uint16_t *x,
                             const uint16_t *wr, const float *bias, const uint8_t *w13, const uint8_t *s13,
                             const uint8_t *w2, const uint8_t *s2, float *logits, int32_t *idx, float *w,
                             int32_t *offsets, int32_t *sorted_token, int32_t *row_of_slot, uint16_t *h,
                             uint16_t *y, uint16_t *out);
double oracle_e4m3_value(int code);
int oracle_e4m3_encode(double v);
int oracle_act_scale_code(const uint16_t *x, int n);
void oracle_act_quant_fp8(int rows, int K, const uint16_t *x, uint8_t *codes, uint8_t *scales);
void oracle_expert_mlp_w4a8(int nrows, int H, int I, const uint16_t *x, const uint8_t *w13, const uint8_t *s13,
                            const uint8_t *w2, const uint8_t *s2, uint16_t *h_out, uint8_t *hq_codes,
                            uint8_t *hq_scales, uint16_t *y_out);
int oracle_layer_forward_w4a8(int T, int H, int I, int E, int k, int ns, float routed_scale, const uint16_t *x,
                              const uint16_t *wr, const float *bias, const uint8_t *w13, const uint8_t *s13,
                              const uint8_t *w2, const uint8_t *s2, float *logits, int32_t *idx, float *w,
                              int32_t *offsets, int32_t *sorted_token, int32_t *row_of_slot, uint16_t *h,
                              uint8_t *hq_codes, uint8_t *hq_scales, uint16_t *y, uint16_t *out);
void oracle_fp8_block_gemm(int M, int N, int K, const uint16_t *x, const uint8_t *w, const uint8_t *ws,
                           uint16_t *y);
void oracle_set_threads(int n);
int oracle_num_threads(void);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) {
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return rng;
}
/* exact-size allocations, filled with arbitrary bytes */
static void *fill(size_t bytes) {
    uint8_t *p = (uint8_t *)malloc(bytes ? bytes : 1);
    if (!p) exit(3);
    for (size_t i = 0; i < bytes; ++i) p[i] = (uint8_t)next();
    return p;
}
/* bf16 values in [-4, 4): sign, exponent 124..128, any mantissa */
static uint16_t *bf16s(size_t n) {
    uint16_t *p = (uint16_t *)malloc(n * 2);
    for (size_t i = 0; i < n; ++i) {
        const uint64_t r = next();
        p[i] = (uint16_t)(((r & 1) << 15) | ((124 + (r >> 1) % 5) << 7) | ((r >> 8) & 0x7F));
    }
    return p;
}
static uint16_t *fp16_scales(size_t n) {
    uint16_t *p = (uint16_t *)malloc(n * 2);
    for (size_t i = 0; i < n; ++i) p[i] = (uint16_t)(0x2000 | (next() & 0x3FF));
    return p;
}
static uint8_t *ue8m0s(size_t n) {
    uint8_t *p = (uint8_t *)malloc(n);
    for (size_t i = 0; i < n; ++i) p[i] = (uint8_t)(120 + next() % 4);
    return p;
}
static uint8_t *e4m3_codes(size_t n) {  /* finite codes only */
    uint8_t *p = (uint8_t *)malloc(n);
    for (size_t i = 0; i < n; ++i) {
        uint8_t c = (uint8_t)next();
        if ((c & 0x7F) == 0x7F) c ^= 1;
        p[i] = c;
    }
    return p;
}
static float *floats(size_t n, float lo, float hi) {
    float *p = (float *)malloc(n * 4);
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * (float)((next() >> 40) * (1.0 / 16777216.0));
    return p;
}

int main(void) {
    const int T = 9, H = 512, I = 256, E = 16, k = 3, ns = 1, G = E + ns, S = k + ns, R = T * S;
    oracle_set_threads(2);
    int fails = 0;

    /* scalar functions over their whole input domains */
    double acc = 0;
    for (int h = 0; h < 65536; ++h) acc += oracle_fp16_to_f64((uint16_t)h) == 0.0;
    for (int b = 0; b < 256; ++b) acc += oracle_int4_code((uint8_t)b, b & 1);
    for (int c = 0; c < 16; ++c) acc += oracle_fp4_value(c);
    for (int e = 0; e < 255; ++e) acc += oracle_ue8m0(e) > 0;
    for (int c = 0; c < 256; ++c) acc += oracle_e4m3_encode(oracle_e4m3_value(c)) >= 0;
    const double specials[] = {0.0, -0.0, 1e300, -1e300, 448.0, 1e-300, 3.0e38};
    for (int i = 0; i < 7; ++i) acc += oracle_f64_to_bf16(specials[i]) + oracle_e4m3_encode(specials[i]);
    for (int i = 0; i < 4096; ++i) {
        const float y = -200.0f + 0.1f * (float)i;
        acc += oracle_exp(y) + oracle_sigmoid(y);
    }

    /* array functions */
    {
        float *y = floats(1000, -100.0f, 100.0f), *o = (float *)malloc(1000 * 4);
        oracle_exp_array(1000, y, o);
        oracle_sigmoid_array(1000, y, o);
        free(y);
        free(o);
    }
    {
        const int N = 32, K = 256;
        uint8_t *w = (uint8_t *)fill((size_t)N * K / 2);
        uint16_t *s = fp16_scales((size_t)N * K / 128);
        uint8_t *s4 = ue8m0s((size_t)N * K / 32);
        double *out = (double *)malloc(sizeof(double) * N * K);
        oracle_dequant_rows(N, K, w, s, out);
        oracle_dequant_fp4_rows(N, K, w, s4, out);
        free(w); free(s); free(s4); free(out);
    }

    /* the INT4 layer, piece by piece and whole */
    uint16_t *x = bf16s((size_t)T * H), *wr = bf16s((size_t)E * H);
    float *bias = floats(E, -0.1f, 0.1f);
    uint8_t *w13 = (uint8_t *)fill((size_t)G * 2 * I * H / 2), *w2 = (uint8_t *)fill((size_t)G * H * I / 2);
    uint16_t *s13 = fp16_scales((size_t)G * 2 * I * H / 128), *s2 = fp16_scales((size_t)G * H * I / 128);
    float *logits = (float *)malloc(sizeof(float) * T * E), *wts = (float *)malloc(sizeof(float) * T * k);
    int32_t *idx = (int32_t *)malloc(4 * (size_t)T * k), *offsets = (int32_t *)malloc(4 * (size_t)(G + 1));
    int32_t *sorted = (int32_t *)malloc(4 * (size_t)R), *ros = (int32_t *)malloc(4 * (size_t)T * S);
    uint16_t *h = (uint16_t *)malloc(2 * (size_t)R * I), *y = (uint16_t *)malloc(2 * (size_t)R * H);
    uint16_t *out = (uint16_t *)malloc(2 * (size_t)T * H);
    oracle_router_logits(T, H, E, x, wr, logits);
    fails += oracle_select(T, E, k, 1.0f, logits, bias, idx, wts) != 0;
    fails += oracle_permute(T, E, k, ns, idx, offsets, sorted, ros) != 0;
    oracle_expert_mlp(T, H, I, x, w13, s13, w2, s2, h, y);  /* T rows through group 0 */
    oracle_combine(T, H, k, ns, y, ros, wts, out);
    fails += oracle_layer_forward(T, H, I, E, k, ns, 1.0f, x, wr, bias, w13, s13, w2, s2, logits, idx, wts, offsets,
                                  sorted, ros, h, y, out) != 0;
    {   /* an out-of-range expert id is rejected, not indexed */
        int32_t bad[3] = {0, E, 1};
        int32_t *off1 = (int32_t *)malloc(4 * (size_t)(G + 1)), *st1 = (int32_t *)malloc(4 * (size_t)S);
        int32_t *r1 = (int32_t *)malloc(4 * (size_t)S);
        fails += oracle_permute(1, E, k, ns, bad, off1, st1, r1) == 0;
        free(off1); free(st1); free(r1);
    }

    /* the FP4 layer */
    uint8_t *f13 = ue8m0s((size_t)G * 2 * I * H / 32), *f2 = ue8m0s((size_t)G * H * I / 32);
    oracle_expert_mlp_fp4(T, H, I, x, w13, f13, w2, f2, h, y);
    fails += oracle_layer_forward_fp4(T, H, I, E, k, ns, 1.0f, x, wr, bias, w13, f13, w2, f2, logits, idx, wts,
                                      offsets, sorted, ros, h, y, out) != 0;

    /* fp8 activations: quantisation, the W4A8 layer, the FP8_BLOCK GEMM */
    {
        uint8_t *codes = (uint8_t *)malloc((size_t)T * H), *scl = (uint8_t *)malloc((size_t)T * H / 128);
        oracle_act_quant_fp8(T, H, x, codes, scl);
        acc += oracle_act_scale_code(x, 128);
        uint16_t z[128];
        memset(z, 0, sizeof z);
        acc += oracle_act_scale_code(z, 128);
        free(codes);
        free(scl);
    }
    uint8_t *hq = (uint8_t *)malloc((size_t)R * I), *hs = (uint8_t *)malloc((size_t)R * I / 128);
    oracle_expert_mlp_w4a8(T, H, I, x, w13, f13, w2, f2, h, hq, hs, y);
    fails += oracle_layer_forward_w4a8(T, H, I, E, k, ns, 1.0f, x, wr, bias, w13, f13, w2, f2, logits, idx, wts,
                                       offsets, sorted, ros, h, hq, hs, y, out) != 0;
    {
        const int M = 5, N = 256, K = 384;
        uint16_t *a = bf16s((size_t)M * K);
        uint8_t *w = e4m3_codes((size_t)N * K), *ws = ue8m0s((size_t)(N / 128) * (K / 128));
        uint16_t *o = (uint16_t *)malloc(2 * (size_t)M * N);
        oracle_fp8_block_gemm(M, N, K, a, w, ws, o);
        free(a); free(w); free(ws); free(o);
    }
    acc += oracle_num_threads();

    free(x); free(wr); free(bias); free(w13); free(w2); free(s13); free(s2); free(logits); free(wts);
    free(idx); free(offsets); free(sorted); free(ros); free(h); free(y); free(out); free(f13); free(f2);
    free(hq); free(hs);
    printf("oracle sanitizer driver: %d failures (checksum %g)\n", fails, acc);
    return fails ? 1 : 0;
}
