"""moe_route_permute_noalloc (the library's own static scratch, no workspace
argument) against moe_route_permute with a caller workspace: two calls in a
row, the second with fewer tokens, every output bit for bit; sizes past the
static scratch are refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import synth
import w4a16_routed_expert_moe_amd as moe
from gpu_common import say, to_dev_bf16

pytestmark = pytest.mark.gpu

H, E, K, I = 4096, 256, 6, 2048


def _outputs(desc, T, x, wr, bias, noalloc):
    G, R, S = desc.groups, desc.rows(T), desc.top_k + desc.n_shared
    o = dict(logits=torch.full((T, E), -7.0, device="cuda"),
             idx=torch.full((T, K), -7, dtype=torch.int32, device="cuda"),
             w=torch.full((T, K), -7.0, device="cuda"),
             offsets=torch.full((G + 1,), -7, dtype=torch.int32, device="cuda"),
             sorted_token=torch.full((R,), -7, dtype=torch.int32, device="cuda"),
             row_of_slot=torch.full((T, S), -7, dtype=torch.int32, device="cuda"))
    args = (desc, T, x, wr, bias, o["logits"], o["idx"], o["w"], o["offsets"], o["sorted_token"],
            o["row_of_slot"])
    if noalloc:
        moe.moe_route_permute_noalloc(*args)
    else:
        ws = torch.zeros(moe.moe_workspace_bytes(desc, T), dtype=torch.uint8, device="cuda")
        moe.moe_route_permute(*args, ws)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in o.items()}


def test_noalloc_matches_the_workspace_entry_point_twice_in_a_row():
    desc = moe.MoeLayerDesc.make(H, I, E, K, 1)
    for T, seed in ((3000, 3), (3, 4)):  # three chunks of the sort, then the one-launch small batch
        say("noalloc route+permute T=%d" % T)
        x = to_dev_bf16(synth.make_x(T, H, seed))
        wr = to_dev_bf16(synth.make_router(E, H, seed))
        bias = torch.from_numpy(synth.make_bias(E, seed)).cuda()
        ref = _outputs(desc, T, x, wr, bias, noalloc=False)
        got = _outputs(desc, T, x, wr, bias, noalloc=True)
        for k in ref:
            assert np.array_equal(got[k].view(np.uint32), ref[k].view(np.uint32)), "%s differs at T=%d" % (k, T)
        say("  T=%d: all outputs bit-identical" % T)


def test_noalloc_refuses_more_tokens_than_its_scratch_holds():
    # through the C ABI directly: the library checks T before it reads any
    # pointer or enqueues anything
    import ctypes
    desc = moe.MoeLayerDesc.make(H, I, E, K, 1)
    buf = torch.zeros(1024, dtype=torch.int32, device="cuda")
    p = ctypes.c_void_p(buf.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    L = moe._lib.lib()
    T = moe._lib.MOE_NOALLOC_MAX_TOKENS + 1
    assert L.moe_route_permute_noalloc(ctypes.byref(desc), T, *[p] * 9, s) == 7  # MOE_ERR_WORKSPACE
    assert L.moe_route_permute_noalloc(ctypes.byref(desc), 0, *[None] * 9, s) == 0
    torch.cuda.synchronize()
    assert int(buf.abs().sum().item()) == 0
    say("  T=%d refused with MOE_ERR_WORKSPACE" % T)
