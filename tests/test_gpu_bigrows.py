"""GPU parity: the grouped GEMMs on an activation matrix of more than 2^32
elements (2.25M rows x K = 2048), the size the ABI admits for the down
projection of 250K tokens (R = T * 9 rows).  The LDS-tiled kernels address a
row of A by its element offset; checked rows on both sides of row 2^21 (where
row * K passes 2^32) must read their own row.  Every other row of A is zero,
so a row read from a wrapped offset would show as a zero or a wrong output.

Only the checked rows of A are filled, from the seeded generator (and, for
W4A8, quantised by the oracle); the expected rows are the oracle's
dequantised weights times those rows in fp64."""
import numpy as np
import pytest
import torch

import oracle
import synth
import w4a16_routed_expert_moe_amd as moe
from gpu_common import TOL, bf16_to_np_bits, rel_err, say

pytestmark = pytest.mark.gpu

T, K = 250_000, 2048
DESC = moe.MoeLayerDesc.make(hidden=4096, inter=K, n_routed=8, top_k=8, n_shared=1)
G, R = DESC.groups, DESC.rows(T)
ROWS = [5, 1_000_003, 1 << 21, (1 << 21) + 9, R - 1]  # 2^21 * 2048 = 2^32


def _group_offsets():
    off = np.full(G + 1, R, np.int32)
    off[0] = 0  # every row in group 0
    return torch.from_numpy(off).cuda()


def _x_rows():
    return synth.make_x(len(ROWS), K, seed=31)  # bf16 bits [rows][K]


def _check(out, N, exp):
    got = bf16_to_np_bits(out[ROWS].reshape(len(ROWS), N))
    e = rel_err(got, exp)
    say("  rows %s rel err %.2e" % (ROWS, e))
    assert e <= TOL


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.empty_cache()


def test_int4_tiled_rows_past_2_32_elements():
    N = 128  # the LDS-tiled kernel (N % 128 == 0)
    assert R * K > 1 << 32 and R >= moe.MOE_TILED_MIN_TOKENS
    w = synth.int4_codes(7, 0, 0, 0, N, K)
    s = synth.fp16_scales(7, 0, 0, 1, N, K)
    canon = np.zeros((G, N, K // 2), np.uint8)
    canon[0] = w
    scales = np.zeros((G, N, K // 128), np.float16)
    scales[0] = s
    packed = torch.empty(G * N * K // 2, dtype=torch.uint8, device="cuda")
    moe.moe_w4a16_prepack(G, N, K, torch.from_numpy(canon.reshape(-1)).cuda(), packed)
    xr = _x_rows()
    a = torch.zeros((R, K), dtype=torch.bfloat16, device="cuda")
    a[ROWS] = torch.from_numpy(xr.view(np.int16)).view(torch.bfloat16).cuda()
    out = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
    moe.moe_w4a16_grouped_gemm(DESC, T, a, None, 0, None, N, K, packed, torch.from_numpy(scales).cuda(),
                               _group_offsets(), moe.MOE_ACT_NONE, out)
    torch.cuda.synchronize()
    wd = oracle.dequant(w, scales[0])
    exp = synth.f32_to_bf16_bits((synth.bf16_bits_to_f32(xr).astype(np.float64) @ wd.T).astype(np.float32))
    _check(out, N, exp)


def test_fp4_wide_rows_past_2_32_elements():
    N = 512  # the 512-wide FP4 kernel
    w = synth.int4_codes(7, 0, 0, 2, N, K)
    s = synth.ue8m0_scales(7, 0, 0, 3, N, K)
    canon = np.zeros((G, N, K // 2), np.uint8)
    canon[0] = w
    scales = np.full((G, N, K // 32), 127, np.uint8)
    scales[0] = s
    packed = torch.empty(G * N * K // 2, dtype=torch.uint8, device="cuda")
    moe.moe_mxfp4_prepack(G, N, K, torch.from_numpy(canon.reshape(-1)).cuda(), packed)
    xr = _x_rows()
    a = torch.zeros((R, K), dtype=torch.bfloat16, device="cuda")
    a[ROWS] = torch.from_numpy(xr.view(np.int16)).view(torch.bfloat16).cuda()
    out = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
    moe.moe_mxfp4_grouped_gemm(DESC, T, a, None, 0, N, K, packed, torch.from_numpy(scales).cuda(),
                               _group_offsets(), moe.MOE_ACT_NONE, out)
    torch.cuda.synchronize()
    wd = oracle.dequant_fp4(w, s)
    exp = synth.f32_to_bf16_bits((synth.bf16_bits_to_f32(xr).astype(np.float64) @ wd.T).astype(np.float32))
    _check(out, N, exp)


def test_w4a8_rows_past_2_32_elements():
    N = 512  # the MX kernel's 512-wide FP4 tiles
    w = synth.int4_codes(7, 0, 0, 2, N, K)
    s = synth.ue8m0_scales(7, 0, 0, 3, N, K)
    canon = np.zeros((G, N, K // 2), np.uint8)
    canon[0] = w
    scales = np.full((G, N, K // 32), 127, np.uint8)
    scales[0] = s
    packed = torch.empty(G * N * K // 2, dtype=torch.uint8, device="cuda")
    moe.moe_mxfp4_prepack(G, N, K, torch.from_numpy(canon.reshape(-1)).cuda(), packed)
    codes, cs = oracle.act_quant_fp8(_x_rows())
    a = torch.zeros((R, K), dtype=torch.uint8, device="cuda")
    a_s = torch.full((R, K // 128), 127, dtype=torch.uint8, device="cuda")
    a[ROWS] = torch.from_numpy(codes).cuda()
    a_s[ROWS] = torch.from_numpy(cs).cuda()
    out = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
    moe.moe_w4a8_grouped_gemm(DESC, T, a, a_s, None, 0, N, K, packed, torch.from_numpy(scales).cuda(),
                              _group_offsets(), moe.MOE_ACT_NONE, out)
    torch.cuda.synchronize()
    lut = np.array([oracle.e4m3_value(c) for c in range(256)], np.float64)
    av = lut[codes] * np.repeat(np.exp2(cs.astype(np.float64) - 127.0), 128, axis=1)
    wd = oracle.dequant_fp4(w, s)
    exp = synth.f32_to_bf16_bits((av @ wd.T).astype(np.float32))
    _check(out, N, exp)
