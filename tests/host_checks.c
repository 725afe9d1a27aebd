/* host_checks.c -- test infrastructure: drives the host-side argument checks
 * of every entry point in include/moe_w4a16.h, for an AddressSanitizer /
 * UndefinedBehaviorSanitizer build of the library's host code
 * (tests/test_sanitizers.py).  Every call here must be rejected by the checks
 * (or be a T = 0 no-op), so nothing reaches the HIP runtime: the device
 * pointers are placeholders that are never dereferenced.  Exit status 0 when
 * every call returned the documented status. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe_w4a16.h"

static int fails = 0;
#define EXPECT(call, want)                                                                    \
    do {                                                                                      \
        moe_status got_ = (call);                                                             \
        if (got_ != (want)) {                                                                 \
            printf("line %d: %s returned %d (%s), expected %d\n", __LINE__, #call, (int)got_, \
                   moe_status_str(got_), (int)(want));                                        \
            ++fails;                                                                          \
        }                                                                                     \
    } while (0)

int main(void) {
    /* placeholders: aligned, never dereferenced (every call below fails its
       checks before anything is enqueued) */
    void *P = (void *)(uintptr_t)0x10000, *U = (void *)(uintptr_t)0x10002;  /* aligned / misaligned */
    const uint16_t *x = (const uint16_t *)P;
    float *f = (float *)P;
    int32_t *i32 = (int32_t *)P;
    uint16_t *b16 = (uint16_t *)P;
    uint8_t *u8 = (uint8_t *)P;

    moe_layer_desc d;
    memset(&d, 0, sizeof d);
    d.hidden = 4096; d.inter = 2048; d.n_routed = 256; d.top_k = 6; d.n_shared = 1; d.group_size = 128;
    d.routed_scale = 1.0f;
    moe_layer_desc bad = d;

    /* descriptor limits */
    EXPECT(moe_route(NULL, 1, x, x, f, f, i32, f, NULL), MOE_ERR_NULL);
    bad.hidden = 300; EXPECT(moe_route(&bad, 1, x, x, f, f, i32, f, NULL), MOE_ERR_SHAPE); bad = d;
    bad.inter = 100; EXPECT(moe_route(&bad, 1, x, x, f, f, i32, f, NULL), MOE_ERR_SHAPE); bad = d;
    bad.n_routed = 0; EXPECT(moe_route(&bad, 1, x, x, f, f, i32, f, NULL), MOE_ERR_SHAPE); bad = d;
    bad.n_routed = 257; EXPECT(moe_route(&bad, 1, x, x, f, f, i32, f, NULL), MOE_ERR_SHAPE); bad = d;
    bad.top_k = 9; EXPECT(moe_route(&bad, 1, x, x, f, f, i32, f, NULL), MOE_ERR_SHAPE); bad = d;
    bad.n_shared = 2; EXPECT(moe_route(&bad, 1, x, x, f, f, i32, f, NULL), MOE_ERR_SHAPE); bad = d;
    bad.group_size = 64; EXPECT(moe_route(&bad, 1, x, x, f, f, i32, f, NULL), MOE_ERR_UNSUPPORTED); bad = d;
    bad.routed_scale = 0.0f / 0.0f; EXPECT(moe_route(&bad, 1, x, x, f, f, i32, f, NULL), MOE_ERR_SHAPE); bad = d;

    /* tokens, nulls, alignment, T = 0 */
    EXPECT(moe_route(&d, -1, x, x, f, f, i32, f, NULL), MOE_ERR_SHAPE);
    EXPECT(moe_route(&d, MOE_MAX_TOKENS + 1, x, x, f, f, i32, f, NULL), MOE_ERR_SHAPE);
    EXPECT(moe_route(&d, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL), MOE_OK);
    EXPECT(moe_route(&d, 3, NULL, x, f, f, i32, f, NULL), MOE_ERR_NULL);
    EXPECT(moe_route(&d, 3, (const uint16_t *)U, x, f, f, i32, f, NULL), MOE_ERR_ALIGN);

    /* workspace */
    if (moe_workspace_bytes(&d, 0) == 0 || moe_workspace_bytes(NULL, 1) != 0) ++fails;
    if (moe_workspace_bytes(&d, 5000) <= moe_workspace_bytes(&d, 1000)) ++fails;
    EXPECT(moe_permute(&d, 2000, i32, i32, i32, i32, P, 16, NULL), MOE_ERR_WORKSPACE);
    EXPECT(moe_permute(&d, 2000, i32, i32, i32, i32, NULL, 0, NULL), MOE_ERR_NULL);
    EXPECT(moe_permute(&d, 2000, i32, i32, i32, i32, U, 1 << 20, NULL), MOE_ERR_ALIGN);
    EXPECT(moe_permute(&d, 0, NULL, NULL, NULL, NULL, NULL, 0, NULL), MOE_OK);
    EXPECT(moe_permute(&d, 5, NULL, i32, i32, i32, NULL, 0, NULL), MOE_ERR_NULL);
    EXPECT(moe_route_permute(&d, 4, x, x, f, f, i32, f, i32, i32, i32, NULL, 0, NULL), MOE_ERR_NULL);
    EXPECT(moe_route_permute(&d, 4, x, x, f, f, i32, f, i32, i32, i32, P, 8, NULL), MOE_ERR_WORKSPACE);
    EXPECT(moe_route_permute(&d, -2, x, x, f, f, i32, f, i32, i32, i32, P, 1 << 20, NULL), MOE_ERR_SHAPE);
    EXPECT(moe_route_permute_noalloc(&d, MOE_NOALLOC_MAX_TOKENS + 1, x, x, f, f, i32, f, i32, i32, i32, NULL),
           MOE_ERR_WORKSPACE);
    EXPECT(moe_route_permute_noalloc(&d, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL), MOE_OK);
    EXPECT(moe_route_permute_noalloc(NULL, 1, x, x, f, f, i32, f, i32, i32, i32, NULL), MOE_ERR_NULL);

    /* grouped GEMMs */
    EXPECT(moe_w4a16_grouped_gemm(&d, 8, x, i32, 8, NULL, 4096, 4096, u8, b16, i32, 7, b16, NULL),
           MOE_ERR_UNSUPPORTED);
    EXPECT(moe_w4a16_grouped_gemm(&d, 8, x, i32, 8, NULL, 4000, 4096, u8, b16, i32, MOE_ACT_NONE, b16, NULL),
           MOE_ERR_SHAPE);
    EXPECT(moe_w4a16_grouped_gemm(&d, 8, x, i32, 8, NULL, 4096, 8192, u8, b16, i32, MOE_ACT_NONE, b16, NULL),
           MOE_ERR_SHAPE);
    EXPECT(moe_w4a16_grouped_gemm(&d, 8, x, i32, 0, NULL, 4096, 4096, u8, b16, i32, MOE_ACT_NONE, b16, NULL),
           MOE_ERR_SHAPE);
    EXPECT(moe_w4a16_grouped_gemm(&d, 8, x, i32, 8, NULL, 4096, 4096, NULL, b16, i32, MOE_ACT_NONE, b16, NULL),
           MOE_ERR_NULL);
    EXPECT(moe_w4a16_grouped_gemm(&d, 8, (const uint16_t *)U, i32, 8, NULL, 4096, 4096, u8, b16, i32,
                                  MOE_ACT_NONE, b16, NULL), MOE_ERR_ALIGN);
    EXPECT(moe_w4a16_grouped_gemm(&d, 0, NULL, NULL, 0, NULL, 4096, 4096, NULL, NULL, NULL, MOE_ACT_NONE, NULL,
                                  NULL), MOE_OK);
    EXPECT(moe_mxfp4_grouped_gemm(&d, 8, x, i32, 8, 4096, 100, u8, u8, i32, MOE_ACT_NONE, b16, NULL),
           MOE_ERR_SHAPE);
    EXPECT(moe_mxfp4_grouped_gemm(&d, 8, x, i32, 8, 4096, 4096, u8, NULL, i32, MOE_ACT_NONE, b16, NULL),
           MOE_ERR_NULL);
    EXPECT(moe_w4a8_grouped_gemm(&d, 8, u8, u8, i32, 8, 4000, 4096, u8, u8, i32, MOE_ACT_NONE, b16, NULL),
           MOE_ERR_SHAPE);
    EXPECT(moe_w4a8_grouped_gemm(&d, 8, u8, u8, i32, 8, 4096, 8192, u8, u8, i32, MOE_ACT_NONE, b16, NULL),
           MOE_ERR_SHAPE);
    EXPECT(moe_w4a8_grouped_gemm(&d, 8, u8, NULL, i32, 8, 4096, 4096, u8, u8, i32, MOE_ACT_NONE, b16, NULL),
           MOE_ERR_NULL);
    EXPECT(moe_fp8_block_gemm(8, 4096, 4100, u8, u8, u8, u8, b16, NULL), MOE_ERR_SHAPE);
    EXPECT(moe_fp8_block_gemm(0, 4096, 4096, NULL, NULL, NULL, NULL, NULL, NULL), MOE_OK);
    EXPECT(moe_fp8_block_gemm(8, 4096, 4096, (const uint8_t *)U, u8, u8, u8, b16, NULL), MOE_ERR_ALIGN);
    EXPECT(moe_act_quant_fp8(4, 100, x, u8, u8, NULL), MOE_ERR_SHAPE);
    EXPECT(moe_act_quant_fp8(4, 128, x, NULL, u8, NULL), MOE_ERR_NULL);
    EXPECT(moe_act_quant_fp8_dequant(4, 100, x, u8, u8, b16, NULL), MOE_ERR_SHAPE);
    EXPECT(moe_act_quant_fp8_dequant(4, 128, x, u8, u8, NULL, NULL), MOE_ERR_NULL);
    EXPECT(moe_act_quant_fp8_dequant(4, 128, x, u8, u8, (uint16_t *)U, NULL), MOE_ERR_ALIGN);
    EXPECT(moe_act_quant_fp8_dequant(4, 128, x, u8, u8, b16, NULL), MOE_ERR_SHAPE);  /* deq overlaps a */
    EXPECT(moe_act_quant_fp8_dequant(4, 128, x, u8, u8, b16 + 4 * 128 - 8, NULL), MOE_ERR_SHAPE);
    EXPECT(moe_act_quant_fp8_dequant(0, 128, NULL, NULL, NULL, NULL, NULL), MOE_OK);
    EXPECT(moe_row_sums(4, 100, x, f, NULL), MOE_ERR_SHAPE);
    EXPECT(moe_row_sums(4, 128, NULL, f, NULL), MOE_ERR_NULL);

    /* combine, fused paths, decode */
    EXPECT(moe_combine(&d, 4, NULL, i32, f, b16, NULL), MOE_ERR_NULL);
    EXPECT(moe_combine(&d, 0, NULL, NULL, NULL, NULL, NULL), MOE_OK);
    EXPECT(moe_w4a16_down_combine(&d, MOE_DOWN_COMBINE_MAX_TOKENS + 1, b16, u8, b16, i32, f, i32, b16, NULL),
           MOE_ERR_UNSUPPORTED);
    EXPECT(moe_w4a16_down_combine(&d, 2, b16, NULL, b16, i32, f, i32, b16, NULL), MOE_ERR_NULL);
    EXPECT(moe_w4a16_decode_token(NULL, x, x, f, u8, b16, u8, b16, f, i32, f, i32, i32, i32, b16, b16, i32, NULL),
           MOE_ERR_NULL);
    EXPECT(moe_w4a16_decode_token(&d, x, x, f, u8, b16, u8, b16, f, i32, f, i32, i32, i32, b16, b16, NULL, NULL),
           MOE_ERR_NULL);
    EXPECT(moe_mxfp4_decode_token(&d, x, x, f, u8, u8, u8, u8, f, i32, f, i32, i32, i32, b16, b16, NULL, NULL),
           MOE_ERR_NULL);

    /* prepacks and generators */
    EXPECT(moe_w4a16_prepack(1, 100, 4096, u8, u8, NULL), MOE_ERR_SHAPE);
    EXPECT(moe_w4a16_prepack(1, 128, 4096, u8, u8, NULL), MOE_ERR_SHAPE);  /* in place: overlapping */
    EXPECT(moe_mxfp4_prepack(1, 128, 4096, NULL, u8, NULL), MOE_ERR_NULL);
    EXPECT(moe_fp8_prepack(100, 4096, u8, u8, NULL), MOE_ERR_SHAPE);
    EXPECT(moe_gen_int4_codes(1, 0, 0, -1, 0, 128, 4096, u8, NULL), MOE_ERR_SHAPE);
    EXPECT(moe_gen_int4_codes(1, 0, 0, 1, 0, 128, 4096, NULL, NULL), MOE_ERR_NULL);
    EXPECT(moe_gen_fp16_scales(1, 0, 0, 1, 0, 128, 4096, NULL, NULL), MOE_ERR_NULL);
    EXPECT(moe_gen_ue8m0_scales(1, 0, 0, -1, 0, 128, 4096, u8, NULL), MOE_ERR_SHAPE);
    EXPECT(moe_gen_ue8m0_scales(1, 0, 0, 0, 0, 128, 4096, NULL, NULL), MOE_OK);

    /* status strings for every code and one past them */
    for (int s = 0; s <= 8; ++s)
        if (!moe_status_str((moe_status)s) || !moe_status_str((moe_status)s)[0]) ++fails;
    if (moe_abi_version() <= 0) ++fails;

    printf("host checks: %d failures\n", fails);
    return fails ? 1 : 0;
}
