"""ctypes binding of ``libmoe_w4a16.so``: the same entry points, argument
marshalling only.

Each wrapper checks the torch tensors it is given (device, dtype, contiguity,
size) so that the C library, which sees only raw pointers, is never handed a
buffer smaller than the shapes imply; then it passes ``data_ptr()`` and the
stream handle through.  Every computation happens in the HIP kernels.  If the
library is missing this module raises at import-use time -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_w4a16.so")

MOE_ACT_NONE = 0
MOE_ACT_SWIGLU = 1
MOE_MAX_TOKENS = 1 << 20
MOE_TILED_MIN_TOKENS = 384
MOE_DOWN_COMBINE_MAX_TOKENS = 4
MOE_DECODE_WORKSPACE_BYTES = 131072
MOE_NOALLOC_MAX_TOKENS = 65536
MOE_NOALLOC_WS_BYTES = 82176
ABI_VERSION = 10

STATUS = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_UNSUPPORTED",
          4: "MOE_ERR_ALIGN", 5: "MOE_ERR_LAUNCH", 6: "MOE_ERR_DEVICE", 7: "MOE_ERR_WORKSPACE"}

# every symbol include/moe_w4a16.h declares
EXPORTS = ("moe_workspace_bytes", "moe_route", "moe_permute", "moe_route_permute", "moe_route_permute_noalloc", "moe_w4a16_grouped_gemm", "moe_row_sums",
           "moe_w4a16_down_combine", "moe_w4a16_decode_token", "moe_w4a16_decode_token_supported", "moe_combine", "moe_w4a16_prepack", "moe_gen_int4_codes", "moe_gen_fp16_scales",
           "moe_mxfp4_grouped_gemm", "moe_mxfp4_prepack", "moe_gen_ue8m0_scales", "moe_mxfp4_decode_token", "moe_w4a8_decode_token",
           "moe_act_quant_fp8", "moe_act_quant_fp8_dequant", "moe_w4a8_grouped_gemm", "moe_fp8_block_gemm", "moe_fp8_prepack",
           "moe_status_str", "moe_abi_version")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s -> %s (%s)" % (fn, STATUS.get(status, status), msg))
        self.status = status


class MoeLayerDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_routed", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("routed_scale", ctypes.c_float)]

    @classmethod
    def make(cls, hidden, inter, n_routed, top_k, n_shared=1, routed_scale=1.0, group_size=128):
        return cls(hidden, inter, n_routed, top_k, n_shared, group_size, routed_scale)

    @property
    def groups(self) -> int:
        return self.n_routed + self.n_shared

    def rows(self, T: int) -> int:
        return T * (self.top_k + self.n_shared)


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe_w4a16.so is not built (run __graft_entry__.build() or "
                               "python w4a16_routed_expert_moe_amd/build.py); there is no fallback")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, u64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
        D = ctypes.POINTER(MoeLayerDesc)
        sigs = {
            "moe_route": [D, i32, P, P, P, P, P, P, P],
            "moe_permute": [D, i32, P, P, P, P, P, SZ, P],
            "moe_route_permute": [D, i32, P, P, P, P, P, P, P, P, P, P, SZ, P],
            "moe_route_permute_noalloc": [D, i32, P, P, P, P, P, P, P, P, P, P],
            "moe_w4a16_grouped_gemm": [D, i32, P, P, i32, P, i32, i32, P, P, P, i32, P, P],
            "moe_row_sums": [i32, i32, P, P, P],
            "moe_w4a16_down_combine": [D, i32, P, P, P, P, P, P, P, P],
            "moe_w4a16_decode_token": [D, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P],
            "moe_w4a16_decode_token_supported": [D],
            "moe_combine": [D, i32, P, P, P, P, P],
            "moe_w4a16_prepack": [i32, i32, i32, P, P, P],
            "moe_gen_int4_codes": [u64, i32, i32, i32, i32, i32, i32, P, P],
            "moe_gen_fp16_scales": [u64, i32, i32, i32, i32, i32, i32, P, P],
            "moe_mxfp4_grouped_gemm": [D, i32, P, P, i32, i32, i32, P, P, P, i32, P, P],
            "moe_mxfp4_prepack": [i32, i32, i32, P, P, P],
            "moe_mxfp4_decode_token": [D, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P],
            "moe_w4a8_decode_token": [D, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P],
            "moe_gen_ue8m0_scales": [u64, i32, i32, i32, i32, i32, i32, P, P],
            "moe_act_quant_fp8": [i32, i32, P, P, P, P],
            "moe_act_quant_fp8_dequant": [i32, i32, P, P, P, P, P],
            "moe_w4a8_grouped_gemm": [D, i32, P, P, P, i32, i32, i32, P, P, P, i32, P, P],
            "moe_fp8_block_gemm": [i32, i32, i32, P, P, P, P, P, P],
            "moe_fp8_prepack": [i32, i32, P, P, P],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.moe_workspace_bytes.argtypes = [D, i32]
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_abi_version.argtypes = []
        L.moe_abi_version.restype = ctypes.c_int32
        if L.moe_abi_version() != ABI_VERSION:
            raise RuntimeError("libmoe_w4a16.so has ABI version %d, this binding expects %d (rebuild)"
                               % (L.moe_abi_version(), ABI_VERSION))
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise MoeError(fn, status, lib().moe_status_str(status).decode())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    return ctypes.c_void_p(int(stream))


def _ptr(t, name, dtype, numel, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.numel() < numel:
        raise ValueError("%s holds %d elements, needs %d" % (name, t.numel(), numel))
    return ctypes.c_void_p(t.data_ptr())


# ------------------------------------------------------------------ entry points
def moe_route(desc: MoeLayerDesc, T: int, x, w_router, gate_bias, logits, topk_idx, topk_w,
              stream=None):
    H, E, k = desc.hidden, desc.n_routed, desc.top_k
    _check("moe_route", lib().moe_route(
        ctypes.byref(desc), T, _ptr(x, "x", torch.bfloat16, T * H),
        _ptr(w_router, "w_router", torch.bfloat16, E * H), _ptr(gate_bias, "gate_bias", torch.float32, E),
        _ptr(logits, "logits", torch.float32, T * E), _ptr(topk_idx, "topk_idx", torch.int32, T * k),
        _ptr(topk_w, "topk_w", torch.float32, T * k), _stream(stream)))


def moe_workspace_bytes(desc: MoeLayerDesc, T: int) -> int:
    """Bytes of the workspace moe_permute / moe_route_permute need at T tokens."""
    return int(lib().moe_workspace_bytes(ctypes.byref(desc), T))


def _ws(ws, name="ws"):
    """(pointer, bytes) of a uint8 device workspace tensor, or (None, 0)."""
    if ws is None:
        return None, 0
    return _ptr(ws, name, torch.uint8, 0), ws.numel()


def moe_permute(desc: MoeLayerDesc, T: int, topk_idx, group_offsets, sorted_token, row_of_slot,
                ws=None, stream=None):
    G, R, S = desc.groups, desc.rows(T), desc.top_k + desc.n_shared
    wp, wb = _ws(ws)
    _check("moe_permute", lib().moe_permute(
        ctypes.byref(desc), T, _ptr(topk_idx, "topk_idx", torch.int32, T * desc.top_k),
        _ptr(group_offsets, "group_offsets", torch.int32, G + 1),
        _ptr(sorted_token, "sorted_token", torch.int32, R),
        _ptr(row_of_slot, "row_of_slot", torch.int32, T * S), wp, wb, _stream(stream)))


def moe_route_permute(desc: MoeLayerDesc, T: int, x, w_router, gate_bias, logits, topk_idx, topk_w,
                      group_offsets, sorted_token, row_of_slot, ws, stream=None):
    H, E, k = desc.hidden, desc.n_routed, desc.top_k
    G, R, S = desc.groups, desc.rows(T), desc.top_k + desc.n_shared
    _check("moe_route_permute", lib().moe_route_permute(
        ctypes.byref(desc), T, _ptr(x, "x", torch.bfloat16, T * H),
        _ptr(w_router, "w_router", torch.bfloat16, E * H), _ptr(gate_bias, "gate_bias", torch.float32, E),
        _ptr(logits, "logits", torch.float32, T * E), _ptr(topk_idx, "topk_idx", torch.int32, T * k),
        _ptr(topk_w, "topk_w", torch.float32, T * k),
        _ptr(group_offsets, "group_offsets", torch.int32, G + 1),
        _ptr(sorted_token, "sorted_token", torch.int32, R),
        _ptr(row_of_slot, "row_of_slot", torch.int32, T * S), *_ws(ws), _stream(stream)))


def moe_route_permute_noalloc(desc: MoeLayerDesc, T: int, x, w_router, gate_bias, logits, topk_idx,
                              topk_w, group_offsets, sorted_token, row_of_slot, stream=None):
    """moe_route_permute with the library's own static scratch (no workspace)."""
    H, E, k = desc.hidden, desc.n_routed, desc.top_k
    G, R, S = desc.groups, desc.rows(T), desc.top_k + desc.n_shared
    _check("moe_route_permute_noalloc", lib().moe_route_permute_noalloc(
        ctypes.byref(desc), T, _ptr(x, "x", torch.bfloat16, T * H),
        _ptr(w_router, "w_router", torch.bfloat16, E * H), _ptr(gate_bias, "gate_bias", torch.float32, E),
        _ptr(logits, "logits", torch.float32, T * E), _ptr(topk_idx, "topk_idx", torch.int32, T * k),
        _ptr(topk_w, "topk_w", torch.float32, T * k),
        _ptr(group_offsets, "group_offsets", torch.int32, G + 1),
        _ptr(sorted_token, "sorted_token", torch.int32, R),
        _ptr(row_of_slot, "row_of_slot", torch.int32, T * S), _stream(stream)))


def moe_w4a16_grouped_gemm(desc: MoeLayerDesc, T: int, a, a_gather, n_src: int, a_sums, N: int, K: int,
                           w_packed, w_scales, group_offsets, act: int, out, stream=None):
    G, R = desc.groups, desc.rows(T)
    a_rows = n_src if a_gather is not None else R
    out_cols = N // 2 if act == MOE_ACT_SWIGLU else N
    _check("moe_w4a16_grouped_gemm", lib().moe_w4a16_grouped_gemm(
        ctypes.byref(desc), T, _ptr(a, "a", torch.bfloat16, a_rows * K),
        _ptr(a_gather, "a_gather", torch.int32, R, optional=True), n_src,
        _ptr(a_sums, "a_sums", torch.float32, a_rows * (K // 128), optional=True), N, K,
        _ptr(w_packed, "w_packed", torch.uint8, G * N * K // 2),
        _ptr(w_scales, "w_scales", torch.float16, G * N * (K // 128)),
        _ptr(group_offsets, "group_offsets", torch.int32, G + 1), act,
        _ptr(out, "out", torch.bfloat16, R * out_cols), _stream(stream)))


def moe_mxfp4_grouped_gemm(desc: MoeLayerDesc, T: int, a, a_gather, n_src: int, N: int, K: int,
                           w_packed, w_scales, group_offsets, act: int, out, stream=None):
    G, R = desc.groups, desc.rows(T)
    a_rows = n_src if a_gather is not None else R
    out_cols = N // 2 if act == MOE_ACT_SWIGLU else N
    _check("moe_mxfp4_grouped_gemm", lib().moe_mxfp4_grouped_gemm(
        ctypes.byref(desc), T, _ptr(a, "a", torch.bfloat16, a_rows * K),
        _ptr(a_gather, "a_gather", torch.int32, R, optional=True), n_src, N, K,
        _ptr(w_packed, "w_packed", torch.uint8, G * N * K // 2),
        _ptr(w_scales, "w_scales", torch.uint8, G * N * (K // 32)),
        _ptr(group_offsets, "group_offsets", torch.int32, G + 1), act,
        _ptr(out, "out", torch.bfloat16, R * out_cols), _stream(stream)))


def moe_row_sums(rows: int, K: int, a, sums, stream=None):
    _check("moe_row_sums", lib().moe_row_sums(
        rows, K, _ptr(a, "a", torch.bfloat16, rows * K),
        _ptr(sums, "sums", torch.float32, rows * (K // 128)), _stream(stream)))


def moe_w4a16_down_combine(desc: MoeLayerDesc, T: int, h, w_packed, w_scales, topk_idx, topk_w,
                           row_of_slot, out, stream=None):
    H, I, G, R, S = desc.hidden, desc.inter, desc.groups, desc.rows(T), desc.top_k + desc.n_shared
    _check("moe_w4a16_down_combine", lib().moe_w4a16_down_combine(
        ctypes.byref(desc), T, _ptr(h, "h", torch.bfloat16, R * I),
        _ptr(w_packed, "w_packed", torch.uint8, G * H * I // 2),
        _ptr(w_scales, "w_scales", torch.float16, G * H * (I // 128)),
        _ptr(topk_idx, "topk_idx", torch.int32, T * desc.top_k),
        _ptr(topk_w, "topk_w", torch.float32, T * desc.top_k),
        _ptr(row_of_slot, "row_of_slot", torch.int32, T * S),
        _ptr(out, "out", torch.bfloat16, T * H), _stream(stream)))


def moe_w4a16_decode_token(desc: MoeLayerDesc, x, w_router, gate_bias, w13_packed, w13_scales, w2_packed,
                           w2_scales, logits, topk_idx, topk_w, group_offsets, sorted_token, row_of_slot,
                           h, out, workspace, stream=None):
    H, I, E, k = desc.hidden, desc.inter, desc.n_routed, desc.top_k
    G, S = desc.groups, desc.top_k + desc.n_shared
    _check("moe_w4a16_decode_token", lib().moe_w4a16_decode_token(
        ctypes.byref(desc), _ptr(x, "x", torch.bfloat16, H),
        _ptr(w_router, "w_router", torch.bfloat16, E * H), _ptr(gate_bias, "gate_bias", torch.float32, E),
        _ptr(w13_packed, "w13_packed", torch.uint8, G * 2 * I * H // 2),
        _ptr(w13_scales, "w13_scales", torch.float16, G * 2 * I * (H // 128)),
        _ptr(w2_packed, "w2_packed", torch.uint8, G * H * I // 2),
        _ptr(w2_scales, "w2_scales", torch.float16, G * H * (I // 128)),
        _ptr(logits, "logits", torch.float32, E), _ptr(topk_idx, "topk_idx", torch.int32, k),
        _ptr(topk_w, "topk_w", torch.float32, k), _ptr(group_offsets, "group_offsets", torch.int32, G + 1),
        _ptr(sorted_token, "sorted_token", torch.int32, S), _ptr(row_of_slot, "row_of_slot", torch.int32, S),
        _ptr(h, "h", torch.bfloat16, S * I), _ptr(out, "out", torch.bfloat16, H),
        _ptr(workspace, "workspace", torch.int32, MOE_DECODE_WORKSPACE_BYTES // 4), _stream(stream)))


def moe_mxfp4_decode_token(desc: MoeLayerDesc, x, w_router, gate_bias, w13_packed, w13_scales, w2_packed,
                           w2_scales, logits, topk_idx, topk_w, group_offsets, sorted_token, row_of_slot,
                           h, out, workspace, stream=None):
    H, I, E, k = desc.hidden, desc.inter, desc.n_routed, desc.top_k
    G, S = desc.groups, desc.top_k + desc.n_shared
    _check("moe_mxfp4_decode_token", lib().moe_mxfp4_decode_token(
        ctypes.byref(desc), _ptr(x, "x", torch.bfloat16, H),
        _ptr(w_router, "w_router", torch.bfloat16, E * H), _ptr(gate_bias, "gate_bias", torch.float32, E),
        _ptr(w13_packed, "w13_packed", torch.uint8, G * 2 * I * H // 2),
        _ptr(w13_scales, "w13_scales", torch.uint8, G * 2 * I * (H // 32)),
        _ptr(w2_packed, "w2_packed", torch.uint8, G * H * I // 2),
        _ptr(w2_scales, "w2_scales", torch.uint8, G * H * (I // 32)),
        _ptr(logits, "logits", torch.float32, E), _ptr(topk_idx, "topk_idx", torch.int32, k),
        _ptr(topk_w, "topk_w", torch.float32, k), _ptr(group_offsets, "group_offsets", torch.int32, G + 1),
        _ptr(sorted_token, "sorted_token", torch.int32, S), _ptr(row_of_slot, "row_of_slot", torch.int32, S),
        _ptr(h, "h", torch.bfloat16, S * I), _ptr(out, "out", torch.bfloat16, H),
        _ptr(workspace, "workspace", torch.int32, MOE_DECODE_WORKSPACE_BYTES // 4), _stream(stream)))


def moe_w4a8_decode_token(desc: MoeLayerDesc, x, w_router, gate_bias, w13_packed, w13_scales, w2_packed,
                           w2_scales, logits, topk_idx, topk_w, group_offsets, sorted_token, row_of_slot,
                           h, out, workspace, stream=None):
    """moe_mxfp4_decode_token with x and h quantised to e4m3 per 128 for the expert GEMMs (W4A8)."""
    H, I, E, k = desc.hidden, desc.inter, desc.n_routed, desc.top_k
    G, S = desc.groups, desc.top_k + desc.n_shared
    _check("moe_w4a8_decode_token", lib().moe_w4a8_decode_token(
        ctypes.byref(desc), _ptr(x, "x", torch.bfloat16, H),
        _ptr(w_router, "w_router", torch.bfloat16, E * H), _ptr(gate_bias, "gate_bias", torch.float32, E),
        _ptr(w13_packed, "w13_packed", torch.uint8, G * 2 * I * H // 2),
        _ptr(w13_scales, "w13_scales", torch.uint8, G * 2 * I * (H // 32)),
        _ptr(w2_packed, "w2_packed", torch.uint8, G * H * I // 2),
        _ptr(w2_scales, "w2_scales", torch.uint8, G * H * (I // 32)),
        _ptr(logits, "logits", torch.float32, E), _ptr(topk_idx, "topk_idx", torch.int32, k),
        _ptr(topk_w, "topk_w", torch.float32, k), _ptr(group_offsets, "group_offsets", torch.int32, G + 1),
        _ptr(sorted_token, "sorted_token", torch.int32, S), _ptr(row_of_slot, "row_of_slot", torch.int32, S),
        _ptr(h, "h", torch.bfloat16, S * I), _ptr(out, "out", torch.bfloat16, H),
        _ptr(workspace, "workspace", torch.int32, MOE_DECODE_WORKSPACE_BYTES // 4), _stream(stream)))


def moe_w4a16_decode_token_supported(desc: MoeLayerDesc) -> int:
    """The status moe_w4a16_decode_token would return for `desc` on the current device (0 = supported)."""
    return int(lib().moe_w4a16_decode_token_supported(ctypes.byref(desc)))


def moe_combine(desc: MoeLayerDesc, T: int, y, row_of_slot, topk_w, out, stream=None):
    H, R, S = desc.hidden, desc.rows(T), desc.top_k + desc.n_shared
    _check("moe_combine", lib().moe_combine(
        ctypes.byref(desc), T, _ptr(y, "y", torch.bfloat16, R * H),
        _ptr(row_of_slot, "row_of_slot", torch.int32, T * S),
        _ptr(topk_w, "topk_w", torch.float32, T * desc.top_k), _ptr(out, "out", torch.bfloat16, T * H),
        _stream(stream)))


def moe_w4a16_prepack(n_groups: int, N: int, K: int, w_canonical, w_packed, stream=None):
    n = n_groups * N * K // 2
    _check("moe_w4a16_prepack", lib().moe_w4a16_prepack(
        n_groups, N, K, _ptr(w_canonical, "w_canonical", torch.uint8, n),
        _ptr(w_packed, "w_packed", torch.uint8, n), _stream(stream)))


def moe_mxfp4_prepack(n_groups: int, N: int, K: int, w_canonical, w_packed, stream=None):
    n = n_groups * N * K // 2
    _check("moe_mxfp4_prepack", lib().moe_mxfp4_prepack(
        n_groups, N, K, _ptr(w_canonical, "w_canonical", torch.uint8, n),
        _ptr(w_packed, "w_packed", torch.uint8, n), _stream(stream)))


def moe_gen_ue8m0_scales(seed: int, layer: int, group0: int, n_groups: int, kind: int, N: int, K: int,
                         out, stream=None):
    _check("moe_gen_ue8m0_scales", lib().moe_gen_ue8m0_scales(
        seed, layer, group0, n_groups, kind, N, K,
        _ptr(out, "out", torch.uint8, n_groups * N * (K // 32)), _stream(stream)))


def moe_gen_int4_codes(seed: int, layer: int, group0: int, n_groups: int, kind: int, N: int, K: int,
                       out, stream=None):
    _check("moe_gen_int4_codes", lib().moe_gen_int4_codes(
        seed, layer, group0, n_groups, kind, N, K,
        _ptr(out, "out", torch.uint8, n_groups * N * K // 2), _stream(stream)))


def moe_gen_fp16_scales(seed: int, layer: int, group0: int, n_groups: int, kind: int, N: int, K: int,
                        out, stream=None):
    _check("moe_gen_fp16_scales", lib().moe_gen_fp16_scales(
        seed, layer, group0, n_groups, kind, N, K,
        _ptr(out, "out", torch.float16, n_groups * N * (K // 128)), _stream(stream)))


def moe_status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def moe_abi_version() -> int:
    return lib().moe_abi_version()


# ------------------------------------------------------------------ fp8 activations
def moe_act_quant_fp8(rows: int, K: int, a, codes, scales, stream=None):
    _check("moe_act_quant_fp8", lib().moe_act_quant_fp8(
        rows, K, _ptr(a, "a", torch.bfloat16, rows * K), _ptr(codes, "codes", torch.uint8, rows * K),
        _ptr(scales, "scales", torch.uint8, rows * (K // 128)), _stream(stream)))


def moe_act_quant_fp8_dequant(rows: int, K: int, a, codes, scales, deq, stream=None):
    _check("moe_act_quant_fp8_dequant", lib().moe_act_quant_fp8_dequant(
        rows, K, _ptr(a, "a", torch.bfloat16, rows * K), _ptr(codes, "codes", torch.uint8, rows * K),
        _ptr(scales, "scales", torch.uint8, rows * (K // 128)), _ptr(deq, "deq", torch.bfloat16, rows * K),
        _stream(stream)))


def moe_w4a8_grouped_gemm(desc: MoeLayerDesc, T: int, a, a_scales, a_gather, n_src: int, N: int, K: int,
                          w_packed, w_scales, group_offsets, act: int, out, stream=None):
    G, R = desc.groups, desc.rows(T)
    a_rows = n_src if a_gather is not None else R
    out_cols = N // 2 if act == MOE_ACT_SWIGLU else N
    _check("moe_w4a8_grouped_gemm", lib().moe_w4a8_grouped_gemm(
        ctypes.byref(desc), T, _ptr(a, "a", torch.uint8, a_rows * K),
        _ptr(a_scales, "a_scales", torch.uint8, a_rows * (K // 128)),
        _ptr(a_gather, "a_gather", torch.int32, R, optional=True), n_src, N, K,
        _ptr(w_packed, "w_packed", torch.uint8, G * N * K // 2),
        _ptr(w_scales, "w_scales", torch.uint8, G * N * (K // 32)),
        _ptr(group_offsets, "group_offsets", torch.int32, G + 1), act,
        _ptr(out, "out", torch.bfloat16, R * out_cols), _stream(stream)))


def moe_fp8_block_gemm(M: int, N: int, K: int, a, a_scales, w_packed, w_scales, out, stream=None):
    _check("moe_fp8_block_gemm", lib().moe_fp8_block_gemm(
        M, N, K, _ptr(a, "a", torch.uint8, M * K), _ptr(a_scales, "a_scales", torch.uint8, M * (K // 128)),
        _ptr(w_packed, "w_packed", torch.uint8, N * K),
        _ptr(w_scales, "w_scales", torch.uint8, (N // 128) * (K // 128)),
        _ptr(out, "out", torch.bfloat16, M * N), _stream(stream)))


def moe_fp8_prepack(N: int, K: int, w_canonical, w_packed, stream=None):
    _check("moe_fp8_prepack", lib().moe_fp8_prepack(
        N, K, _ptr(w_canonical, "w_canonical", torch.uint8, N * K), _ptr(w_packed, "w_packed", torch.uint8, N * K),
        _stream(stream)))
