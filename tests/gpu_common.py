"""Shared set-up for the GPU parity tests: build a layer on the device from
the seeded generators, run it through the C ABI, and compute the oracle's
answer on the same inputs.  The HIP side and the oracle share only the input
generators (``synth``)."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle
import synth
import w4a16_routed_expert_moe_amd as moe

TOL = 2e-2  # max |out - ref| <= TOL * max |ref|  (bf16 activations, fp32 accumulation)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_to_np_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


class Case:
    """One layer instance: shape, inputs on host and device, device weights."""

    def __init__(self, name, T=None, H=None, E=None, k=None, I=None, n_shared=None, seed=0, layer=0,
                 routing=None, weights="device", routed_scale=1.0, fmt="int4", w4a8=False):
        w = dict(synth.WORKLOADS[name]) if name in synth.WORKLOADS else {}
        self.name = name
        self.T = T if T is not None else w["T"]
        self.H = H if H is not None else w["H"]
        self.E = E if E is not None else w["E"]
        self.k = k if k is not None else w["k"]
        self.I = I if I is not None else w["I"]
        self.ns = n_shared if n_shared is not None else w.get("n_shared", 1)
        self.seed, self.layer = seed, layer
        self.G = self.E + self.ns
        routing = routing or w.get("routing", "iid")
        self.bias = synth.make_bias(self.E, seed, layer)
        if routing == "zipf":
            self.x, self.wr = synth.make_zipf_router(self.T, self.H, self.E, seed)
        elif routing == "uniform":
            self.wr = synth.make_router(self.E, self.H, seed, layer)
            self.x = synth.make_uniform_x(self.T, self.H, self.wr, self.bias, seed, layer)
        else:
            self.x = synth.make_x(self.T, self.H, seed)
            self.wr = synth.make_router(self.E, self.H, seed, layer)
        self.desc = moe.MoeLayerDesc.make(self.H, self.I, self.E, self.k, self.ns, routed_scale)
        self.routed_scale = routed_scale
        self.fmt = fmt
        say("case %s: T=%d H=%d E=%d k=%d I=%d ns=%d seed=%d layer=%d fmt=%s%s" %
            (name, self.T, self.H, self.E, self.k, self.I, self.ns, seed, layer, fmt, " w4a8" if w4a8 else ""))
        if weights == "device":
            self.experts = moe.generate_weights(seed, layer, self.G, self.H, self.I, fmt=fmt)
        else:
            w13, s13, w2, s2 = self.stacked_weights()
            self.experts = moe.upload_weights(w13, s13, w2, s2, fmt=fmt)
        self.w4a8 = w4a8
        self.layer_obj = moe.MoELayer(self.desc, to_dev_bf16(self.wr), torch.from_numpy(self.bias).cuda(),
                                      self.experts, w4a8=w4a8)
        self.xd = to_dev_bf16(self.x)
        self.buf = moe.Buffers(self.desc, self.T, fp8=w4a8)

    def stacked_weights(self):
        gen = synth.stacked_expert_weights if self.fmt == "int4" else synth.stacked_fp4_expert_weights
        return gen(self.seed, self.layer, self.G, self.H, self.I)

    @functools.lru_cache(maxsize=None)
    def group_weights(self, g):
        gen = synth.expert_weights if self.fmt == "int4" else synth.fp4_expert_weights
        return gen(self.seed, self.layer, g, self.H, self.I)

    def run(self):
        out = self.layer_obj.forward(self.xd, self.buf)
        torch.cuda.synchronize()
        return out

    def oracle_routing(self):
        logits = oracle.router_logits(self.x, self.wr)
        idx, w = oracle.select(logits, self.bias, self.k, self.routed_scale)
        offsets, sorted_token, row_of_slot = oracle.permute(idx, self.E, self.ns)
        return dict(logits=logits, idx=idx, w=w, offsets=offsets, sorted_token=sorted_token,
                    row_of_slot=row_of_slot)

    def gpu_routing(self):
        b = self.buf
        return dict(logits=b.logits.cpu().numpy(), idx=b.topk_idx.cpu().numpy(),
                    w=b.topk_w.cpu().numpy(), offsets=b.group_offsets.cpu().numpy(),
                    sorted_token=b.sorted_token.cpu().numpy(), row_of_slot=b.row_of_slot.cpu().numpy())

    def oracle_tokens(self, tokens, ref_routing):
        return oracle.token_outputs(tokens, self.x, ref_routing["idx"], ref_routing["w"],
                                    self.group_weights, self.E, self.ns, fmt=self.fmt)


def assert_routing_equal(got, ref, check_logits=True):
    if check_logits:
        assert np.array_equal(got["logits"].view(np.uint32), ref["logits"].view(np.uint32)), \
            "logits differ in %d places" % int((got["logits"] != ref["logits"]).sum())
    assert np.array_equal(got["idx"], ref["idx"]), "expert indices differ"
    assert np.array_equal(got["w"].view(np.uint32), ref["w"].view(np.uint32)), "routing weights differ"
    assert np.array_equal(got["offsets"], ref["offsets"]), "group offsets differ"
    assert np.array_equal(got["sorted_token"], ref["sorted_token"]), "sorted_token differs"
    assert np.array_equal(got["row_of_slot"], ref["row_of_slot"]), "row_of_slot differs"


def rel_err(out_bits: np.ndarray, ref_bits: np.ndarray) -> float:
    o, r = bits_to_f64(out_bits), bits_to_f64(ref_bits)
    return float(np.max(np.abs(o - r)) / max(np.max(np.abs(r)), 1e-30))
