"""GPU parity of the layer with FP4 expert weights (E2M1 elements, one UE8M0
scale per 32 elements along K) against the oracle, through the C ABI: the
device generator and the FP4 prepack against their documented definitions,
whole layers element by element at small shapes, and sampled tokens at the
full decode and prefill sizes."""
import numpy as np

import oracle
import pytest
import torch

import synth
import w4a16_routed_expert_moe_amd as moe
from gpu_common import TOL, Case, assert_routing_equal, bf16_to_np_bits, rel_err, say
from test_gpu_parity import _check_full

pytestmark = pytest.mark.gpu


def test_mxfp4_device_scale_generator_matches_host():
    for (N, K) in [(256, 4096), (4096, 2048), (48, 96)]:
        say("ue8m0 generator N=%d K=%d" % (N, K))
        out = torch.empty((2, N, K // 32), dtype=torch.uint8, device="cuda")
        moe.moe_gen_ue8m0_scales(0, 3, 5, 2, synth.KIND_S13, N, K, out)
        torch.cuda.synchronize()
        for i in range(2):
            ref = synth.ue8m0_scales(0, 3, 5 + i, synth.KIND_S13, N, K)
            assert np.array_equal(out[i].cpu().numpy(), ref)


def test_mxfp4_prepack_copies_words_into_the_documented_blocks():
    say("fp4 prepack G=2 N=48 K=384")
    G, N, K = 2, 48, 384
    rng = np.random.default_rng(9)
    canon = rng.integers(0, 256, size=(G, N, K // 2), dtype=np.uint8)
    dev = torch.from_numpy(canon.reshape(-1).copy()).cuda()
    out = torch.empty(G * N * K // 2, dtype=torch.uint8, device="cuda")
    moe.moe_mxfp4_prepack(G, N, K, dev, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view("<u4")
    words = canon.reshape(G, N, K // 8, 4).copy().view("<u4").reshape(G, N, K // 8)
    KG, NT = K // 128, N // 16
    exp = np.empty(G * N * K // 8, np.uint32)
    for g in range(G):
        for nt in range(NT):
            for kg in range(KG):
                base = ((g * NT + nt) * KG + kg) * 256
                for l in range(64):
                    n = nt * 16 + l % 16
                    for d in range(4):
                        k0 = kg * 128 + 32 * (l // 16) + 8 * d
                        exp[base + 4 * l + d] = words[g, n, k0 // 8]
    assert np.array_equal(got, exp)


def test_mxfp4_tiny_layer_every_element():
    _check_full(Case("tiny", weights="host", fmt="fp4"))


@pytest.mark.parametrize("shape", [
    dict(T=37, H=1024, E=40, k=3, I=384, n_shared=1),
    dict(T=5, H=512, E=8, k=8, I=128, n_shared=0),
    dict(T=1, H=2048, E=64, k=4, I=256, n_shared=1),
    dict(T=300, H=512, E=256, k=6, I=128, n_shared=1),   # weight-stream kernel
    dict(T=420, H=512, E=256, k=6, I=128, n_shared=1),   # tiled kernel
    dict(T=3, H=1024, E=32, k=4, I=256, n_shared=1),     # 4-row work items, activations preloaded
    dict(T=420, H=1024, E=8, k=3, I=512, n_shared=1),    # 512-wide tiles, K/128 = 8 and 4 (runtime k loop)
    dict(T=400, H=4096, E=8, k=2, I=2048, n_shared=1),   # 512-wide tiles at K = 4096 and 2048
    dict(T=440, H=1024, E=16, k=2, I=512, n_shared=1),   # 512-wide tiles of at most 64 rows
])
def test_mxfp4_ragged_and_edge_shapes_every_element(shape):
    import os
    oracle.set_threads(max(1, min(16, len(os.sched_getaffinity(0)))))
    _check_full(Case("shape", seed=8, weights="host", fmt="fp4", **shape))


def _sampled(case, tokens):
    out = bf16_to_np_bits(case.run())
    ref = case.oracle_routing()
    assert_routing_equal(case.gpu_routing(), ref)
    e = rel_err(out[tokens], case.oracle_tokens(tokens, ref))
    say("  sampled tokens %s rel err %.2e" % (list(tokens), e))
    assert e <= TOL


def test_mxfp4_decode_bs1_full_size():
    _sampled(Case("decode1", fmt="fp4"), [0])


def test_mxfp4_decode_bs64_zipf_full_size():
    _sampled(Case("decode64", fmt="fp4"), [0, 63])


def test_mxfp4_prefill_8192_full_size():
    _sampled(Case("prefill8k", fmt="fp4"), [0, 4097, 8191])


def _fp4_token_case(shape, seed, weights="host"):
    case = Case("shape", T=1, seed=seed, weights=weights, fmt="fp4", **shape)
    assert case.layer_obj.one_launch(1), "the device does not support this decode shape"
    return case


@pytest.mark.parametrize("shape", [
    dict(H=2048, E=64, k=4, I=256, n_shared=1),
    dict(H=2048, E=16, k=8, I=1024, n_shared=0),
    dict(H=2048, E=128, k=6, I=1536, n_shared=1),
    dict(H=4096, E=32, k=2, I=512, n_shared=1),
])
def test_mxfp4_decode_token_every_element(shape):
    # the one-launch step with FP4 experts: routing bit-exact, h and out
    # within tolerance of the oracle, and close to the separate launches
    from test_gpu_parity import _full_oracle
    case = _fp4_token_case(shape, seed=23)
    outs = []
    for _ in range(3):
        outs.append(bf16_to_np_bits(case.run()).copy())
        ws = case.buf.decode_ws[:5].cpu().numpy()
        assert ws[3] == 0, "a wait timed out"
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    ref = _full_oracle(case)
    assert_routing_equal(case.gpu_routing(), ref)
    eh, eo = rel_err(bf16_to_np_bits(case.buf.h), ref["h"]), rel_err(outs[0], ref["out"])
    case.layer_obj.fuse_token = False
    sep = bf16_to_np_bits(case.run()).copy()
    es = rel_err(outs[0], sep)
    say("  rel err h %.2e out %.2e; vs separate launches %.2e" % (eh, eo, es))
    assert eh <= TOL and eo <= TOL and es <= TOL


def test_mxfp4_decode_token_full_size_seed31():
    case = _fp4_token_case(dict(H=4096, E=256, k=6, I=2048, n_shared=1), seed=31, weights="device")
    _sampled(case, [0])
