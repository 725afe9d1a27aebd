"""One routed-expert MoE layer on the GPU: buffers plus the five library calls.

``MoELayer.forward`` enqueues, on one stream and with no host synchronisation:
route -> permute -> gate/up grouped GEMM with SwiGLU -> down grouped GEMM ->
combine (from MOE_TILED_MIN_TOKENS tokens on, each GEMM is preceded by the
row sums of its input, which the tiled GEMM takes for its offset correction;
up to MOE_DOWN_COMBINE_MAX_TOKENS tokens the down GEMM and the combine are one
call, which keeps y in fp32 and never stores it; a single token takes the
whole layer in one call, moe_w4a16_decode_token, where the device supports
its shape).  Experts in FP4 (``ExpertWeights.fmt == "fp4"``, the release's
own expert format) take moe_mxfp4_decode_token for a single token and
otherwise moe_mxfp4_grouped_gemm for both GEMMs and the separate combine.  Buffers are allocated once per token count and reused,
so the sequence can be captured in a HIP graph.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib as L

KIND_W13, KIND_W2, KIND_S13, KIND_S2 = 0, 1, 2, 3


@dataclass
class ExpertWeights:
    """Expert weights of all G groups, resident in HBM.

    w13: INT4 codes of the gate/up projections in the streamed layout,
         G*2I*H/2 bytes; s13: fp16 [G][2I][H/128].
    w2:  INT4 codes of the down projection, G*H*I/2 bytes; s2: fp16 [G][H][I/128].
    fmt "fp4": E2M1 codes in the FP4 layout, s13 UE8M0 [G][2I][H/32], s2 UE8M0 [G][H][I/32].
    """
    w13: torch.Tensor
    s13: torch.Tensor
    w2: torch.Tensor
    s2: torch.Tensor
    fmt: str = "int4"

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.w13, self.s13, self.w2, self.s2))


def prepack(canonical: torch.Tensor, n_groups: int, N: int, K: int, stream=None,
            fmt: str = "int4") -> torch.Tensor:
    """Canonical codes (device, uint8) -> the streamed layout (a new tensor)."""
    out = torch.empty(n_groups * N * K // 2, dtype=torch.uint8, device=canonical.device)
    fn = L.moe_w4a16_prepack if fmt == "int4" else L.moe_mxfp4_prepack
    fn(n_groups, N, K, canonical.reshape(-1), out, stream)
    return out


def upload_weights(w13, s13, w2, s2, device="cuda", fmt: str = "int4") -> ExpertWeights:
    """Host canonical arrays (numpy, stacked over groups) -> resident ExpertWeights."""
    G, twoI = w13.shape[0], w13.shape[1]
    H = w13.shape[2] * 2
    I = twoI // 2
    gs = 128 if fmt == "int4" else 32  # elements per scale along K
    c13 = torch.from_numpy(w13.reshape(-1).copy()).to(device)
    c2 = torch.from_numpy(w2.reshape(-1).copy()).to(device)
    return ExpertWeights(
        w13=prepack(c13, G, 2 * I, H, fmt=fmt),
        s13=torch.from_numpy(s13.reshape(G, 2 * I, H // gs).copy()).to(device),
        w2=prepack(c2, G, H, I, fmt=fmt),
        s2=torch.from_numpy(s2.reshape(G, H, I // gs).copy()).to(device), fmt=fmt)


def generate_weights(seed: int, layer: int, G: int, H: int, I: int, device="cuda",
                     scratch: torch.Tensor | None = None, fmt: str = "int4") -> ExpertWeights:
    """Synthetic weights of one layer drawn on the device (counter-based
    SplitMix64, the same streams as ``synth.expert_weights`` or, for ``fmt``
    "fp4", ``synth.fp4_expert_weights``), then prepacked.
    ``scratch`` (uint8, >= G*2I*H/2 bytes) may be passed to avoid a temporary."""
    if fmt == "fp4":
        return _generate_fp4(seed, layer, G, H, I, device, scratch)
    n13 = G * 2 * I * H // 2
    n2 = G * H * I // 2
    if scratch is None or scratch.numel() < n13:
        scratch = torch.empty(n13, dtype=torch.uint8, device=device)
    w13 = torch.empty(n13, dtype=torch.uint8, device=device)
    w2 = torch.empty(n2, dtype=torch.uint8, device=device)
    s13 = torch.empty((G, 2 * I, H // 128), dtype=torch.float16, device=device)
    s2 = torch.empty((G, H, I // 128), dtype=torch.float16, device=device)
    L.moe_gen_int4_codes(seed, layer, 0, G, KIND_W13, 2 * I, H, scratch)
    L.moe_w4a16_prepack(G, 2 * I, H, scratch[:n13], w13)
    L.moe_gen_int4_codes(seed, layer, 0, G, KIND_W2, H, I, scratch)
    L.moe_w4a16_prepack(G, H, I, scratch[:n2], w2)
    L.moe_gen_fp16_scales(seed, layer, 0, G, KIND_S13, 2 * I, H, s13)
    L.moe_gen_fp16_scales(seed, layer, 0, G, KIND_S2, H, I, s2)
    return ExpertWeights(w13=w13, s13=s13, w2=w2, s2=s2)


def _generate_fp4(seed, layer, G, H, I, device, scratch) -> ExpertWeights:
    n13 = G * 2 * I * H // 2
    n2 = G * H * I // 2
    if scratch is None or scratch.numel() < n13:
        scratch = torch.empty(n13, dtype=torch.uint8, device=device)
    w13 = torch.empty(n13, dtype=torch.uint8, device=device)
    w2 = torch.empty(n2, dtype=torch.uint8, device=device)
    s13 = torch.empty((G, 2 * I, H // 32), dtype=torch.uint8, device=device)
    s2 = torch.empty((G, H, I // 32), dtype=torch.uint8, device=device)
    L.moe_gen_int4_codes(seed, layer, 0, G, KIND_W13, 2 * I, H, scratch)
    L.moe_mxfp4_prepack(G, 2 * I, H, scratch[:n13], w13)
    L.moe_gen_int4_codes(seed, layer, 0, G, KIND_W2, H, I, scratch)
    L.moe_mxfp4_prepack(G, H, I, scratch[:n2], w2)
    L.moe_gen_ue8m0_scales(seed, layer, 0, G, KIND_S13, 2 * I, H, s13)
    L.moe_gen_ue8m0_scales(seed, layer, 0, G, KIND_S2, H, I, s2)
    return ExpertWeights(w13=w13, s13=s13, w2=w2, s2=s2, fmt="fp4")


class Buffers:
    """Device buffers of one forward pass at token count T."""

    def __init__(self, desc: L.MoeLayerDesc, T: int, device="cuda", fp8: bool = False):
        H, I, E, k, ns = desc.hidden, desc.inter, desc.n_routed, desc.top_k, desc.n_shared
        G, R = desc.groups, desc.rows(T)
        self.T = T
        self.logits = torch.empty((T, E), dtype=torch.float32, device=device)
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=device)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.group_offsets = torch.empty(G + 1, dtype=torch.int32, device=device)
        self.sorted_token = torch.empty(R, dtype=torch.int32, device=device)
        self.row_of_slot = torch.empty((T, k + ns), dtype=torch.int32, device=device)
        self.h = torch.empty((R, I), dtype=torch.bfloat16, device=device)
        self.y = torch.empty((R, H), dtype=torch.bfloat16, device=device)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=device)
        # row sums over 128-wide k groups of the two GEMM inputs (x, h), used
        # by the tiled GEMM from MOE_TILED_MIN_TOKENS tokens on
        self.tiled = T >= L.MOE_TILED_MIN_TOKENS
        self.x_sums = torch.empty((T, H // 128) if self.tiled else (0,), dtype=torch.float32, device=device)
        self.h_sums = torch.empty((R, I // 128) if self.tiled else (0,), dtype=torch.float32, device=device)
        # from MOE_TILED_MIN_TOKENS tokens with one shared expert, while the
        # routed groups average fewer than 96 rows (the GEMMs' 64-row tiles):
        # the shared expert's GEMMs (rows R-T.., in token order) go on a side
        # stream beside the routing, with 128-row tiles of their own (43-layer
        # stack at 2048 tokens: 1.33 -> 1.30 ms per layer INT4, 1.21 -> 1.18 ms
        # FP4).  With larger groups the extra launches cost more than the
        # overlap gives (8192 tokens: 4.26 -> 4.29 ms INT4)
        self.split = self.tiled and ns == 1 and T * k < 96 * E
        if self.split:
            self.side = torch.cuda.Stream(device=device)
            self.ev_sums = torch.cuda.Event()
            self.shared_offsets = torch.tensor([0, T], dtype=torch.int32, device=device)
        # scratch of moe_route_permute / moe_permute (zero before the first
        # call: its header holds the small-batch arrival counter)
        self.ws = torch.zeros(max(L.moe_workspace_bytes(desc, T), 256), dtype=torch.uint8, device=device)
        # counters of the one-launch decode step (zero; every call leaves them zero)
        self.decode_ws = torch.zeros(L.MOE_DECODE_WORKSPACE_BYTES // 4 if T == 1 else 0,
                                     dtype=torch.int32, device=device)
        # fp8 activations of the W4A8 layer: x and h as e4m3 codes with one
        # UE8M0 scale per 128
        self.fp8 = fp8
        if fp8:
            self.xq = torch.empty((T, H), dtype=torch.uint8, device=device)
            self.xqs = torch.empty((T, H // 128), dtype=torch.uint8, device=device)
            self.hq = torch.empty((R, I), dtype=torch.uint8, device=device)
            self.hqs = torch.empty((R, I // 128), dtype=torch.uint8, device=device)
            # below MOE_TILED_MIN_TOKENS: the quantised x and h as bf16, the
            # operands of the FP4 weight-stream GEMMs
            n = 0 if self.tiled else 1
            self.xdq = torch.empty((T * n, H), dtype=torch.bfloat16, device=device)
            self.hdq = torch.empty((R * n, I), dtype=torch.bfloat16, device=device)

    def check_decode(self) -> None:
        """After the one-launch decode step: wait for the device, then raise
        ``DecodeTimeout`` if a wait of any call since the last check timed out
        (workspace word 3; the outputs of that call and of every later one are
        unspecified).  The workspace is zeroed again before raising, so the
        next call starts clean.  A no-op for buffers without that workspace."""
        if self.decode_ws.numel() <= 3:
            return
        torch.cuda.synchronize(self.decode_ws.device)
        if int(self.decode_ws[3].item()) != 0:
            self.decode_ws.zero_()
            torch.cuda.synchronize(self.decode_ws.device)
            raise DecodeTimeout("a wait of the one-launch decode step timed out (were all of its "
                                "workgroups resident at once?): its outputs are unspecified")


class DecodeTimeout(RuntimeError):
    """The one-launch decode step gave up on a wait; see Buffers.check_decode."""


class MoELayer:
    """Router weight, gate bias and expert weights of one layer."""

    def __init__(self, desc: L.MoeLayerDesc, w_router: torch.Tensor, gate_bias: torch.Tensor,
                 experts: ExpertWeights, fuse_decode: bool = True, fuse_token: bool = True,
                 w4a8: bool = False):
        if w4a8 and experts.fmt != "fp4":
            raise ValueError("the W4A8 layer takes FP4 expert weights")
        self.w4a8 = w4a8
        self.desc = desc
        self.fuse_decode = fuse_decode
        self.fuse_token = fuse_token
        self._token_ok = None
        self.w_router = w_router
        self.gate_bias = gate_bias
        self.experts = experts

    def forward(self, x: torch.Tensor, buf: Buffers, stream=None) -> torch.Tensor:
        d, T = self.desc, buf.T
        H, I = d.hidden, d.inter
        ex = self.experts
        if self.w4a8:
            # W4A8: x and h quantised to e4m3 per token per 128; from
            # MOE_TILED_MIN_TOKENS tokens both GEMMs on the block-scaled
            # fp8 x FP4 matrix cores
            if not buf.fp8:
                raise ValueError("the W4A8 layer needs Buffers(..., fp8=True)")
            if self.one_launch(T):  # a single token: the whole layer in one launch
                L.moe_w4a8_decode_token(d, x, self.w_router, self.gate_bias, ex.w13, ex.s13, ex.w2, ex.s2,
                                        buf.logits, buf.topk_idx, buf.topk_w, buf.group_offsets,
                                        buf.sorted_token, buf.row_of_slot, buf.h, buf.out, buf.decode_ws,
                                        stream)
                return buf.out
            R = d.rows(T)
            L.moe_route_permute(d, T, x, self.w_router, self.gate_bias, buf.logits, buf.topk_idx,
                                buf.topk_w, buf.group_offsets, buf.sorted_token, buf.row_of_slot,
                                buf.ws, stream)
            if not buf.tiled:
                # few tokens: the weight stream bounds the GEMMs, and the
                # quantised operands are exact in bf16, so the FP4
                # weight-stream kernels multiply them (the products are the
                # block-scaled instruction's; only the fp32 summation order
                # differs)
                L.moe_act_quant_fp8_dequant(T, H, x, buf.xq, buf.xqs, buf.xdq, stream)
                L.moe_mxfp4_grouped_gemm(d, T, buf.xdq, buf.sorted_token, T, 2 * I, H, ex.w13, ex.s13,
                                         buf.group_offsets, L.MOE_ACT_SWIGLU, buf.h, stream)
                L.moe_act_quant_fp8_dequant(R, I, buf.h, buf.hq, buf.hqs, buf.hdq, stream)
                L.moe_mxfp4_grouped_gemm(d, T, buf.hdq, None, 0, H, I, ex.w2, ex.s2, buf.group_offsets,
                                         L.MOE_ACT_NONE, buf.y, stream)
                L.moe_combine(d, T, buf.y, buf.row_of_slot, buf.topk_w, buf.out, stream)
                return buf.out
            L.moe_act_quant_fp8(T, H, x, buf.xq, buf.xqs, stream)
            L.moe_w4a8_grouped_gemm(d, T, buf.xq, buf.xqs, buf.sorted_token, T, 2 * I, H, ex.w13, ex.s13,
                                    buf.group_offsets, L.MOE_ACT_SWIGLU, buf.h, stream)
            L.moe_act_quant_fp8(R, I, buf.h, buf.hq, buf.hqs, stream)
            L.moe_w4a8_grouped_gemm(d, T, buf.hq, buf.hqs, None, 0, H, I, ex.w2, ex.s2, buf.group_offsets,
                                    L.MOE_ACT_NONE, buf.y, stream)
            L.moe_combine(d, T, buf.y, buf.row_of_slot, buf.topk_w, buf.out, stream)
            return buf.out
        if buf.split and stream is None:
            return self._forward_split(x, buf)
        if ex.fmt == "fp4" and self.one_launch(T):
            L.moe_mxfp4_decode_token(d, x, self.w_router, self.gate_bias, ex.w13, ex.s13, ex.w2, ex.s2,
                                     buf.logits, buf.topk_idx, buf.topk_w, buf.group_offsets,
                                     buf.sorted_token, buf.row_of_slot, buf.h, buf.out, buf.decode_ws,
                                     stream)
            return buf.out
        if ex.fmt == "fp4":
            L.moe_route_permute(d, T, x, self.w_router, self.gate_bias, buf.logits, buf.topk_idx,
                                buf.topk_w, buf.group_offsets, buf.sorted_token, buf.row_of_slot,
                                buf.ws, stream)
            L.moe_mxfp4_grouped_gemm(d, T, x, buf.sorted_token, T, 2 * I, H, ex.w13, ex.s13,
                                     buf.group_offsets, L.MOE_ACT_SWIGLU, buf.h, stream)
            L.moe_mxfp4_grouped_gemm(d, T, buf.h, None, 0, H, I, ex.w2, ex.s2, buf.group_offsets,
                                     L.MOE_ACT_NONE, buf.y, stream)
            L.moe_combine(d, T, buf.y, buf.row_of_slot, buf.topk_w, buf.out, stream)
            return buf.out
        if self.one_launch(T):
            ex = self.experts
            L.moe_w4a16_decode_token(d, x, self.w_router, self.gate_bias, ex.w13, ex.s13, ex.w2, ex.s2,
                                     buf.logits, buf.topk_idx, buf.topk_w, buf.group_offsets,
                                     buf.sorted_token, buf.row_of_slot, buf.h, buf.out, buf.decode_ws,
                                     stream)
            return buf.out
        L.moe_route_permute(d, T, x, self.w_router, self.gate_bias, buf.logits, buf.topk_idx,
                            buf.topk_w, buf.group_offsets, buf.sorted_token, buf.row_of_slot,
                            buf.ws, stream)
        ex = self.experts
        xs = hs = None
        if buf.tiled:
            xs, hs = buf.x_sums, buf.h_sums
            L.moe_row_sums(T, H, x, xs, stream)
        L.moe_w4a16_grouped_gemm(d, T, x, buf.sorted_token, T, xs, 2 * I, H, ex.w13, ex.s13,
                                 buf.group_offsets, L.MOE_ACT_SWIGLU, buf.h, stream)
        if self.fused_down(T):
            L.moe_w4a16_down_combine(d, T, buf.h, ex.w2, ex.s2, buf.topk_idx, buf.topk_w,
                                     buf.row_of_slot, buf.out, stream)
            return buf.out
        if buf.tiled:
            L.moe_row_sums(d.rows(T), I, buf.h, hs, stream)
        L.moe_w4a16_grouped_gemm(d, T, buf.h, None, 0, hs, H, I, ex.w2, ex.s2, buf.group_offsets,
                                 L.MOE_ACT_NONE, buf.y, stream)
        L.moe_combine(d, T, buf.y, buf.row_of_slot, buf.topk_w, buf.out, stream)
        return buf.out

    def _forward_split(self, x: torch.Tensor, buf: Buffers) -> torch.Tensor:
        """From MOE_TILED_MIN_TOKENS tokens with one shared expert: the shared
        expert's GEMMs need no routing (its group is the last T permuted rows,
        token t at row R-T+t), so they run on a side stream while the main
        stream routes and permutes, then multiplies the routed groups; the
        combine joins the two.  Same kernels, same rows, same results as the
        one-stream path."""
        d, T = self.desc, buf.T
        H, I, E, R = d.hidden, d.inter, d.n_routed, d.rows(T)
        ex = self.experts
        int4 = ex.fmt == "int4"
        routed = L.MoeLayerDesc.make(H, I, E, d.top_k, 0, d.routed_scale)
        shared = L.MoeLayerDesc.make(H, I, 1, 1, 0)
        # group E's weights and scales: the last of the stacked groups
        w13 = ex.w13[E * (ex.w13.numel() // (E + 1)):]
        s13 = ex.s13[E:]
        w2 = ex.w2[E * (ex.w2.numel() // (E + 1)):]
        s2 = ex.s2[E:]
        h_sh, y_sh = buf.h[R - T:], buf.y[R - T:]
        main = torch.cuda.current_stream()
        buf.side.wait_stream(main)  # x is ready
        with torch.cuda.stream(buf.side):
            xs = hs = hs_sh = None
            if int4:
                xs, hs, hs_sh = buf.x_sums, buf.h_sums, buf.h_sums[R - T:]
                L.moe_row_sums(T, H, x, xs)
                buf.ev_sums.record(buf.side)
                L.moe_w4a16_grouped_gemm(shared, T, x, None, 0, xs, 2 * I, H, w13, s13, buf.shared_offsets,
                                         L.MOE_ACT_SWIGLU, h_sh)
                L.moe_row_sums(T, I, h_sh, hs_sh)
                L.moe_w4a16_grouped_gemm(shared, T, h_sh, None, 0, hs_sh, H, I, w2, s2, buf.shared_offsets,
                                         L.MOE_ACT_NONE, y_sh)
            else:
                L.moe_mxfp4_grouped_gemm(shared, T, x, None, 0, 2 * I, H, w13, s13, buf.shared_offsets,
                                         L.MOE_ACT_SWIGLU, h_sh)
                L.moe_mxfp4_grouped_gemm(shared, T, h_sh, None, 0, H, I, w2, s2, buf.shared_offsets,
                                         L.MOE_ACT_NONE, y_sh)
        L.moe_route_permute(d, T, x, self.w_router, self.gate_bias, buf.logits, buf.topk_idx, buf.topk_w,
                            buf.group_offsets, buf.sorted_token, buf.row_of_slot, buf.ws)
        Rr = R - T  # the routed groups' rows
        if int4:
            main.wait_event(buf.ev_sums)  # the row sums of x
            L.moe_w4a16_grouped_gemm(routed, T, x, buf.sorted_token, T, xs, 2 * I, H, ex.w13, ex.s13,
                                     buf.group_offsets, L.MOE_ACT_SWIGLU, buf.h)
            L.moe_row_sums(Rr, I, buf.h, hs)
            L.moe_w4a16_grouped_gemm(routed, T, buf.h, None, 0, hs, H, I, ex.w2, ex.s2, buf.group_offsets,
                                     L.MOE_ACT_NONE, buf.y)
        else:
            L.moe_mxfp4_grouped_gemm(routed, T, x, buf.sorted_token, T, 2 * I, H, ex.w13, ex.s13,
                                     buf.group_offsets, L.MOE_ACT_SWIGLU, buf.h)
            L.moe_mxfp4_grouped_gemm(routed, T, buf.h, None, 0, H, I, ex.w2, ex.s2, buf.group_offsets,
                                     L.MOE_ACT_NONE, buf.y)
        main.wait_stream(buf.side)
        L.moe_combine(d, T, buf.y, buf.row_of_slot, buf.topk_w, buf.out)
        return buf.out

    def one_launch(self, T: int) -> bool:
        """A single token takes the one-launch decode step when the device supports the shape."""
        if T != 1 or not self.fuse_token:
            return False
        if self._token_ok is None:
            self._token_ok = L.moe_w4a16_decode_token_supported(self.desc) == 0
        return self._token_ok

    def fused_down(self, T: int) -> bool:
        """Decode batches take the fused down projection + combine (no y)."""
        return (self.fuse_decode and T <= L.MOE_DOWN_COMBINE_MAX_TOKENS
                and self.desc.inter // 128 in (4, 8, 16, 32))
