"""GPU parity at the full layer shape (hidden 4096, 256 experts top-6 + one
shared, intermediate 2048; "DeepSeek V4 Flash serving hardware", 01 "Sparse
architecture"), element by element over whole expert groups.

The layer runs through the C ABI exactly as the benchmark runs it; then every
h and y value of the chosen groups is compared with the oracle's expert MLP
on the same gathered rows (``oracle.expert_mlp``), so the full K = 4096 / 2048
reductions, every tile position of the tiled kernel (the shared expert's rows
cover all of them at 8192 tokens) and the weight-stream kernel's long k
slices are checked, not only sampled outputs.  Routing and the permutation
are compared bit for bit with the oracle over every token; at the 43-layer
stack on every layer.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
import w4a16_routed_expert_moe_amd as moe
from gpu_common import (TOL, Case, assert_routing_equal, bf16_to_np_bits, bits_to_f64, rel_err,
                        say, to_dev_bf16)

pytestmark = pytest.mark.gpu


def _oracle_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    oracle.set_threads(max(1, min(16, n)))


def _check_groups(case: Case, ref_routing, groups, what):
    """Every h and y value of the listed groups against the oracle's MLP on the
    same permuted rows; returns the largest relative error seen."""
    _oracle_threads()
    off = ref_routing["offsets"]
    st = ref_routing["sorted_token"]
    h_all = bf16_to_np_bits(case.buf.h)
    y_all = bf16_to_np_bits(case.buf.y) if case.buf.y.numel() else None
    mlp = oracle.expert_mlp if case.fmt == "int4" else oracle.expert_mlp_fp4
    worst = 0.0
    for g in groups:
        lo, hi = int(off[g]), int(off[g + 1])
        if hi == lo:
            continue
        h_ref, y_ref = mlp(case.x[st[lo:hi]], *case.group_weights(g))
        eh = rel_err(h_all[lo:hi], h_ref)
        msg = "  %s group %d (%d rows): h rel err %.2e" % (what, g, hi - lo, eh)
        assert eh <= TOL, msg
        worst = max(worst, eh)
        if y_all is not None:
            ey = rel_err(y_all[lo:hi], y_ref)
            msg += ", y rel err %.2e" % ey
            assert ey <= TOL, msg
            worst = max(worst, ey)
        say(msg)
    return worst


def _groups_by_size(offsets, E, picks):
    """Routed groups: the largest, the smallest non-empty and the median one."""
    counts = np.diff(offsets)[:E]
    nz = np.flatnonzero(counts)
    order = nz[np.argsort(counts[nz], kind="stable")]
    sel = {"max": int(order[-1]), "min": int(order[0]), "mid": int(order[len(order) // 2])}
    return [sel[p] for p in picks]


@pytest.mark.parametrize("fmt", ["int4", "fp4"])
def test_prefill8k_whole_groups(fmt):
    # 8192 tokens, uniform routing: the tiled kernel with 128-row tiles.  The
    # shared expert's 8192 rows fill 64 whole tiles; three routed groups add
    # ragged last tiles.
    case = Case("prefill8k", fmt=fmt)
    case.run()
    ref = case.oracle_routing()
    assert_routing_equal(case.gpu_routing(), ref)
    groups = [case.E] + _groups_by_size(ref["offsets"], case.E, ["max", "min", "mid"])
    worst = _check_groups(case, ref, groups, "prefill8k %s" % fmt)
    say("  prefill8k %s: max rel err %.2e over %d groups" % (fmt, worst, len(groups)))


def test_stack43_routing_every_layer():
    # the 43 layers of the stack share x and each have their own router and
    # bias: route + permute of every layer, bit for bit against the oracle
    w = synth.WORKLOADS["stack43"]
    T, H, E, k = w["T"], w["H"], w["E"], w["k"]
    desc = moe.MoeLayerDesc.make(H, w["I"], E, k, 1)
    x = synth.make_x(T, H, 0)
    xd = to_dev_bf16(x)
    buf = moe.Buffers(desc, T)
    _oracle_threads()
    for layer in range(w["layers"]):
        wr = synth.make_router(E, H, 0, layer)
        bias = synth.make_bias(E, 0, layer)
        moe.moe_route_permute(desc, T, xd, to_dev_bf16(wr), torch.from_numpy(bias).cuda(), buf.logits,
                              buf.topk_idx, buf.topk_w, buf.group_offsets, buf.sorted_token,
                              buf.row_of_slot, buf.ws)
        torch.cuda.synchronize()
        logits = oracle.router_logits(x, wr)
        idx, wts = oracle.select(logits, bias, k)
        offsets, st, ros = oracle.permute(idx, E, 1)
        got = dict(logits=buf.logits.cpu().numpy(), idx=buf.topk_idx.cpu().numpy(),
                   w=buf.topk_w.cpu().numpy(), offsets=buf.group_offsets.cpu().numpy(),
                   sorted_token=buf.sorted_token.cpu().numpy(), row_of_slot=buf.row_of_slot.cpu().numpy())
        assert_routing_equal(got, dict(logits=logits, idx=idx, w=wts, offsets=offsets, sorted_token=st,
                                       row_of_slot=ros))
        if layer % 8 == 0 or layer == w["layers"] - 1:
            say("  stack43 layer %d: routing bit-exact (%d experts chosen)" %
                (layer, int((np.diff(offsets)[:E] > 0).sum())))


@pytest.mark.parametrize("layer,fmt", [(0, "int4"), (21, "int4"), (42, "int4"), (21, "fp4")])
def test_stack43_whole_groups(layer, fmt):
    # 2048 tokens: ~58 rows per chosen expert, the tiled kernel with 64-row
    # tiles; the shared expert's 2048 rows and three routed groups
    case = Case("stack43", layer=layer, fmt=fmt)
    case.run()
    ref = case.oracle_routing()
    assert_routing_equal(case.gpu_routing(), ref)
    groups = [case.E] + _groups_by_size(ref["offsets"], case.E, ["max", "min", "mid"])
    worst = _check_groups(case, ref, groups, "stack43 layer %d %s" % (layer, fmt))
    out = bf16_to_np_bits(case.buf.out)
    e = rel_err(out[[0, 1023, 2047]], case.oracle_tokens([0, 1023, 2047], ref))
    say("  stack43 layer %d %s: max group rel err %.2e, sampled out %.2e" % (layer, fmt, worst, e))
    assert e <= TOL


@pytest.mark.parametrize("fmt", ["int4", "fp4"])
def test_decode64_hot_expert_whole_group(fmt):
    # 64 tokens with Zipf-skewed routing: the weight-stream kernel (8-row work
    # items, K/128 = 32 for gate/up and 16 for down); the hottest expert spans
    # several work items, the shared expert all 64 tokens
    case = Case("decode64", fmt=fmt)
    case.run()
    ref = case.oracle_routing()
    assert_routing_equal(case.gpu_routing(), ref)
    hot = _groups_by_size(ref["offsets"], case.E, ["max", "min"])
    worst = _check_groups(case, ref, [case.E] + hot, "decode64 %s" % fmt)
    out = bf16_to_np_bits(case.buf.out)
    toks = list(range(0, 64, 9))
    e = rel_err(out[toks], case.oracle_tokens(toks, ref))
    say("  decode64 %s: max group rel err %.2e, out (%d tokens) %.2e" % (fmt, worst, len(toks), e))
    assert e <= TOL


@pytest.mark.parametrize("fmt", ["int4", "fp4"])
def test_decode1_one_launch_h_and_out(fmt):
    # the one-launch step at full size: all seven h rows (six routed slots and
    # the shared one, in permuted order) against the oracle's MLP, and out
    case = Case("decode1", fmt=fmt)
    assert case.layer_obj.one_launch(1)
    out = bf16_to_np_bits(case.run())
    assert int(case.buf.decode_ws[3].item()) == 0, "a wait timed out"
    ref = case.oracle_routing()
    assert_routing_equal(case.gpu_routing(), ref)
    _oracle_threads()
    mlp = oracle.expert_mlp if fmt == "int4" else oracle.expert_mlp_fp4
    h = bf16_to_np_bits(case.buf.h)
    worst = 0.0
    for g in range(case.G):
        lo, hi = int(ref["offsets"][g]), int(ref["offsets"][g + 1])
        if hi > lo:
            h_ref, _ = mlp(case.x[ref["sorted_token"][lo:hi]], *case.group_weights(g))
            worst = max(worst, rel_err(h[lo:hi], h_ref))
    e = rel_err(out, case.oracle_tokens([0], ref))
    say("  decode1 %s one launch: h rel err %.2e (7 rows), out %.2e" % (fmt, worst, e))
    assert worst <= TOL and e <= TOL


@pytest.mark.parametrize("shape", [
    dict(T=40, H=2048, E=8, k=2, I=1024, n_shared=1),    # stream kernel, 8-row items, K/128 = 16 and 8
    dict(T=64, H=4096, E=16, k=4, I=512, n_shared=1),    # K/128 = 32 for gate/up, ~16 rows per group
    dict(T=17, H=1024, E=4, k=1, I=2048, n_shared=0),    # down K/128 = 16, no shared expert
])
def test_weight_stream_long_k_every_element(shape):
    # every element of h, y and out with the weight-stream kernel's long k
    # slices (the full-size decode shapes' K/128 = 16 and 32)
    case = Case("shape", seed=17, weights="host", **shape)
    case.layer_obj.fuse_decode = False
    out = bf16_to_np_bits(case.run())
    w13, s13, w2, s2 = case.stacked_weights()
    ref = oracle.layer_forward(case.x, case.wr, case.bias, w13, s13, w2, s2, k=case.k, n_shared=case.ns)
    assert_routing_equal(case.gpu_routing(), ref)
    eh = rel_err(bf16_to_np_bits(case.buf.h), ref["h"])
    ey = rel_err(bf16_to_np_bits(case.buf.y), ref["y"])
    eo = rel_err(out, ref["out"])
    say("  rel err h %.2e y %.2e out %.2e" % (eh, ey, eo))
    assert eh <= TOL and ey <= TOL and eo <= TOL
