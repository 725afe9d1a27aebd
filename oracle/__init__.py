"""CPU oracle of the W4A16 routed-expert MoE layer (and of the same layer with
the release's FP4 expert weights) -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it.

The arithmetic lives in ``moe_oracle.c`` (plain C, built with gcc,
``-ffp-contract=off``, no fast-math); this module only builds the library and
marshals numpy arrays.  Pins that tie each function to the pages or to
mathematics are in ``tests/test_oracle_*.py``; every function here is pinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()


def _cpu_has_fma() -> bool:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("flags"):
                    return " fma " in (line + " ")
    except OSError:
        pass
    return False


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with gcc (``force=False``: only if missing)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-Wno-unknown-pragmas"]
    if _cpu_has_fma():
        cmd.append("-mfma")  # hardware fmaf (the oracle's fmaf is correctly rounded either way)
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd += [_SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            L = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            i32, f32, i64 = ctypes.c_int, ctypes.c_float, ctypes.c_int64
            sig = {
                "oracle_fp16_to_f64": (ctypes.c_double, [ctypes.c_uint16]),
                "oracle_f64_to_bf16": (ctypes.c_uint16, [ctypes.c_double]),
                "oracle_int4_code": (i32, [ctypes.c_uint8, i32]),
                "oracle_dequant_rows": (None, [i32, i32, P, P, P]),
                "oracle_fp4_value": (ctypes.c_double, [i32]),
                "oracle_ue8m0": (ctypes.c_double, [i32]),
                "oracle_dequant_fp4_rows": (None, [i32, i32, P, P, P]),
                "oracle_expert_mlp_fp4": (None, [i32, i32, i32, P, P, P, P, P, P, P]),
                "oracle_layer_forward_fp4": (i32, [i32, i32, i32, i32, i32, i32, f32] + [P] * 16),
                "oracle_exp": (f32, [f32]),
                "oracle_sigmoid": (f32, [f32]),
                "oracle_exp_array": (None, [i64, P, P]),
                "oracle_sigmoid_array": (None, [i64, P, P]),
                "oracle_router_logits": (None, [i32, i32, i32, P, P, P]),
                "oracle_select": (i32, [i32, i32, i32, f32, P, P, P, P]),
                "oracle_permute": (i32, [i32, i32, i32, i32, P, P, P, P]),
                "oracle_expert_mlp": (None, [i32, i32, i32, P, P, P, P, P, P, P]),
                "oracle_combine": (None, [i32, i32, i32, i32, P, P, P, P]),
                "oracle_layer_forward": (i32, [i32, i32, i32, i32, i32, i32, f32] + [P] * 16),
                "oracle_e4m3_value": (ctypes.c_double, [i32]),
                "oracle_e4m3_encode": (i32, [ctypes.c_double]),
                "oracle_act_scale_code": (i32, [P, i32]),
                "oracle_act_quant_fp8": (None, [i32, i32, P, P, P]),
                "oracle_expert_mlp_w4a8": (None, [i32, i32, i32, P, P, P, P, P, P, P, P, P]),
                "oracle_layer_forward_w4a8": (i32, [i32, i32, i32, i32, i32, i32, f32] + [P] * 18),
                "oracle_fp8_block_gemm": (None, [i32, i32, i32, P, P, P, P]),
                "oracle_num_threads": (i32, []),
                "oracle_set_threads": (None, [i32]),
            }
            for name, (res, args) in sig.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- scalars
def int4_code(byte: int, high: int) -> int:
    return lib().oracle_int4_code(byte, high)


def fp16_to_f64(bits: int) -> float:
    return lib().oracle_fp16_to_f64(bits)


def f64_to_bf16(x: float) -> int:
    return lib().oracle_f64_to_bf16(x)


def dequant(w: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Canonical codes ``[N][K/2]`` + fp16 scales ``[N][K/128]`` -> fp64 ``[N][K]``."""
    N, K = w.shape[0], w.shape[1] * 2
    out = np.empty((N, K), np.float64)
    lib().oracle_dequant_rows(N, K, _p(_c(w, np.uint8)), _p(_c(s, np.float16)), _p(out))
    return out


def fp4_value(code: int) -> float:
    """E2M1 element ``code`` (0..15) as a number."""
    return lib().oracle_fp4_value(code)


def ue8m0(E: int) -> float:
    """UE8M0 scale byte ``E`` as a number (2^(E-127); NaN for 255)."""
    return lib().oracle_ue8m0(E)


def dequant_fp4(w: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Canonical FP4 codes ``[N][K/2]`` + UE8M0 scales ``[N][K/32]`` -> fp64 ``[N][K]``."""
    N, K = w.shape[0], w.shape[1] * 2
    out = np.empty((N, K), np.float64)
    lib().oracle_dequant_fp4_rows(N, K, _p(_c(w, np.uint8)), _p(_c(s, np.uint8)), _p(out))
    return out


def exp(y) -> np.ndarray:
    y = _c(y, np.float32)
    out = np.empty_like(y)
    lib().oracle_exp_array(y.size, _p(y), _p(out))
    return out


def sigmoid(y) -> np.ndarray:
    y = _c(y, np.float32)
    out = np.empty_like(y)
    lib().oracle_sigmoid_array(y.size, _p(y), _p(out))
    return out


# ---------------------------------------------------------------- routing
def router_logits(x_bits: np.ndarray, wr_bits: np.ndarray) -> np.ndarray:
    x_bits, wr_bits = _c(x_bits, np.uint16), _c(wr_bits, np.uint16)
    T, H = x_bits.shape
    E = wr_bits.shape[0]
    assert H % 512 == 0 and wr_bits.shape[1] == H
    out = np.empty((T, E), np.float32)
    lib().oracle_router_logits(T, H, E, _p(x_bits), _p(wr_bits), _p(out))
    return out


def select(logits: np.ndarray, bias: np.ndarray, k: int, routed_scale: float = 1.0):
    logits, bias = _c(logits, np.float32), _c(bias, np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    rc = lib().oracle_select(T, E, k, routed_scale, _p(logits), _p(bias), _p(idx), _p(w))
    if rc != 0:
        raise ValueError("non-finite routing key")
    return idx, w


def permute(idx: np.ndarray, E: int, n_shared: int = 1):
    idx = _c(idx, np.int32)
    T, k = idx.shape
    G, S = E + n_shared, k + n_shared
    offsets = np.empty(G + 1, np.int32)
    sorted_token = np.empty(T * S, np.int32)
    row_of_slot = np.empty((T, S), np.int32)
    rc = lib().oracle_permute(T, E, k, n_shared, _p(idx), _p(offsets), _p(sorted_token),
                              _p(row_of_slot))
    if rc != 0:
        raise ValueError("expert index out of range")
    return offsets, sorted_token, row_of_slot


# ---------------------------------------------------------------- experts
def expert_mlp(x_bits: np.ndarray, w13, s13, w2, s2):
    """Rows ``x_bits [n][H]`` through one group -> ``(h_bits [n][I], y_bits [n][H])``."""
    x_bits = _c(x_bits, np.uint16)
    n, H = x_bits.shape
    I = w2.shape[1] * 2
    assert w13.shape == (2 * I, H // 2)
    h = np.empty((n, I), np.uint16)
    y = np.empty((n, H), np.uint16)
    lib().oracle_expert_mlp(n, H, I, _p(x_bits), _p(_c(w13, np.uint8)), _p(_c(s13, np.float16)),
                            _p(_c(w2, np.uint8)), _p(_c(s2, np.float16)), _p(h), _p(y))
    return h, y


def expert_mlp_fp4(x_bits: np.ndarray, w13, s13, w2, s2):
    """``expert_mlp`` with FP4 weights (UE8M0 scales ``s13 [2I][H/32]``, ``s2 [H][I/32]``)."""
    x_bits = _c(x_bits, np.uint16)
    n, H = x_bits.shape
    I = w2.shape[1] * 2
    assert w13.shape == (2 * I, H // 2) and s13.shape == (2 * I, H // 32) and s2.shape == (H, I // 32)
    h = np.empty((n, I), np.uint16)
    y = np.empty((n, H), np.uint16)
    lib().oracle_expert_mlp_fp4(n, H, I, _p(x_bits), _p(_c(w13, np.uint8)), _p(_c(s13, np.uint8)),
                                _p(_c(w2, np.uint8)), _p(_c(s2, np.uint8)), _p(h), _p(y))
    return h, y


def combine(y_bits: np.ndarray, row_of_slot: np.ndarray, w: np.ndarray, n_shared: int = 1):
    y_bits, row_of_slot, w = _c(y_bits, np.uint16), _c(row_of_slot, np.int32), _c(w, np.float32)
    T, k = w.shape
    H = y_bits.shape[1]
    out = np.empty((T, H), np.uint16)
    lib().oracle_combine(T, H, k, n_shared, _p(y_bits), _p(row_of_slot), _p(w), _p(out))
    return out


def layer_forward(x_bits, wr_bits, bias, w13, s13, w2, s2, k: int, n_shared: int = 1,
                  routed_scale: float = 1.0, fmt: str = "int4") -> dict:
    """The whole layer (small shapes).  Weights are stacked canonical arrays over G groups;
    ``fmt`` "int4" (fp16 scales per 128) or "fp4" (UE8M0 scales per 32)."""
    x_bits, wr_bits, bias = _c(x_bits, np.uint16), _c(wr_bits, np.uint16), _c(bias, np.float32)
    sdt = np.float16 if fmt == "int4" else np.uint8
    w13, s13, w2, s2 = _c(w13, np.uint8), _c(s13, sdt), _c(w2, np.uint8), _c(s2, sdt)
    T, H = x_bits.shape
    E = wr_bits.shape[0]
    G = E + n_shared
    I = w2.shape[2] * 2
    assert w13.shape[0] == G and w13.shape[1] == 2 * I
    R = T * (k + n_shared)
    o = dict(logits=np.empty((T, E), np.float32), idx=np.empty((T, k), np.int32),
             w=np.empty((T, k), np.float32), offsets=np.empty(G + 1, np.int32),
             sorted_token=np.empty(R, np.int32), row_of_slot=np.empty((T, k + n_shared), np.int32),
             h=np.empty((R, I), np.uint16), y=np.empty((R, H), np.uint16),
             out=np.empty((T, H), np.uint16))
    fwd = lib().oracle_layer_forward if fmt == "int4" else lib().oracle_layer_forward_fp4
    rc = fwd(T, H, I, E, k, n_shared, routed_scale, _p(x_bits), _p(wr_bits),
                                    _p(bias), _p(w13), _p(s13), _p(w2), _p(s2), _p(o["logits"]),
                                    _p(o["idx"]), _p(o["w"]), _p(o["offsets"]),
                                    _p(o["sorted_token"]), _p(o["row_of_slot"]), _p(o["h"]),
                                    _p(o["y"]), _p(o["out"]))
    if rc != 0:
        raise ValueError("oracle_layer_forward failed (%d)" % rc)
    return o


def token_outputs(tokens, x_bits, idx, w, weights_of_group, E: int, n_shared: int = 1,
                  fmt: str = "int4"):
    """Layer output rows for the listed tokens only (large shapes).

    ``idx``/``w`` are the oracle's routing for all tokens; ``weights_of_group(g)``
    returns the canonical ``(w13, s13, w2, s2)`` of group ``g``; ``fmt`` "int4",
    "fp4" or "w4a8" (FP4 weights, fp8 activations).  Each token's
    ``k`` routed rows and its shared row go through ``expert_mlp`` and are
    combined with ``combine``.
    """
    k = idx.shape[1]
    tokens = list(tokens)
    H = x_bits.shape[1]
    rows = {}  # group -> list of tokens
    for t in tokens:
        for j in range(k):
            rows.setdefault(int(idx[t, j]), []).append(t)
        if n_shared:
            rows.setdefault(E, []).append(t)
    y_of = {}
    for g, ts in rows.items():
        if fmt == "w4a8":
            y = expert_mlp_w4a8(x_bits[ts], *weights_of_group(g))[3]
        else:
            _, y = (expert_mlp if fmt == "int4" else expert_mlp_fp4)(x_bits[ts], *weights_of_group(g))
        for i, t in enumerate(ts):
            y_of[(g, t)] = y[i]
    S = k + n_shared
    out = np.empty((len(tokens), H), np.uint16)
    for i, t in enumerate(tokens):
        ys = [y_of[(int(idx[t, j]), t)] for j in range(k)]
        if n_shared:
            ys.append(y_of[(E, t)])
        ymat = np.stack(ys)
        ros = np.arange(S, dtype=np.int32)[None, :]
        out[i] = combine(ymat, ros, w[t:t + 1], n_shared)[0]
    return out


# ---------------------------------------------------------------- fp8 activations
def e4m3_value(code: int) -> float:
    """OCP E4M3FN byte ``code`` as a number (NaN for 0x7F and 0xFF)."""
    return lib().oracle_e4m3_value(code)


def e4m3_encode(v: float) -> int:
    """Nearest E4M3FN code to ``v`` (ties to the even code; +-448 beyond)."""
    return lib().oracle_e4m3_encode(float(v))


def act_scale_code(x_bits: np.ndarray) -> int:
    """UE8M0 code of the activation scale of a block of bf16 values."""
    x_bits = _c(x_bits, np.uint16).reshape(-1)
    return lib().oracle_act_scale_code(_p(x_bits), x_bits.size)


def act_quant_fp8(x_bits: np.ndarray):
    """bf16 ``[rows][K]`` -> (e4m3 codes ``[rows][K]`` u8, UE8M0 scales ``[rows][K/128]`` u8)."""
    x_bits = _c(x_bits, np.uint16)
    rows, K = x_bits.shape
    codes = np.empty((rows, K), np.uint8)
    scales = np.empty((rows, K // 128), np.uint8)
    lib().oracle_act_quant_fp8(rows, K, _p(x_bits), _p(codes), _p(scales))
    return codes, scales


def expert_mlp_w4a8(x_bits: np.ndarray, w13, s13, w2, s2):
    """The W4A8 MLP (FP4 weights as ``expert_mlp_fp4``) ->
    ``(h_bits [n][I], hq_codes [n][I], hq_scales [n][I/128], y_bits [n][H])``."""
    x_bits = _c(x_bits, np.uint16)
    n, H = x_bits.shape
    I = w2.shape[1] * 2
    h = np.empty((n, I), np.uint16)
    hc = np.empty((n, I), np.uint8)
    hs = np.empty((n, I // 128), np.uint8)
    y = np.empty((n, H), np.uint16)
    lib().oracle_expert_mlp_w4a8(n, H, I, _p(x_bits), _p(_c(w13, np.uint8)), _p(_c(s13, np.uint8)),
                                 _p(_c(w2, np.uint8)), _p(_c(s2, np.uint8)), _p(h), _p(hc), _p(hs), _p(y))
    return h, hc, hs, y


def layer_forward_w4a8(x_bits, wr_bits, bias, w13, s13, w2, s2, k: int, n_shared: int = 1,
                       routed_scale: float = 1.0) -> dict:
    """The whole W4A8 layer (stacked FP4 weights as ``layer_forward(fmt="fp4")``)."""
    x_bits, wr_bits, bias = _c(x_bits, np.uint16), _c(wr_bits, np.uint16), _c(bias, np.float32)
    w13, s13, w2, s2 = _c(w13, np.uint8), _c(s13, np.uint8), _c(w2, np.uint8), _c(s2, np.uint8)
    T, H = x_bits.shape
    E = wr_bits.shape[0]
    G = E + n_shared
    I = w2.shape[2] * 2
    R = T * (k + n_shared)
    o = dict(logits=np.empty((T, E), np.float32), idx=np.empty((T, k), np.int32),
             w=np.empty((T, k), np.float32), offsets=np.empty(G + 1, np.int32),
             sorted_token=np.empty(R, np.int32), row_of_slot=np.empty((T, k + n_shared), np.int32),
             h=np.empty((R, I), np.uint16), hq=np.empty((R, I), np.uint8),
             hs=np.empty((R, I // 128), np.uint8), y=np.empty((R, H), np.uint16),
             out=np.empty((T, H), np.uint16))
    rc = lib().oracle_layer_forward_w4a8(T, H, I, E, k, n_shared, routed_scale, _p(x_bits), _p(wr_bits),
                                         _p(bias), _p(w13), _p(s13), _p(w2), _p(s2), _p(o["logits"]),
                                         _p(o["idx"]), _p(o["w"]), _p(o["offsets"]), _p(o["sorted_token"]),
                                         _p(o["row_of_slot"]), _p(o["h"]), _p(o["hq"]), _p(o["hs"]),
                                         _p(o["y"]), _p(o["out"]))
    if rc != 0:
        raise ValueError("oracle_layer_forward_w4a8 failed (%d)" % rc)
    return o


def fp8_block_gemm(x_bits: np.ndarray, w_codes: np.ndarray, w_scales: np.ndarray) -> np.ndarray:
    """FP8_BLOCK GEMM: bf16 ``x [M][K]``, e4m3 ``W [N][K]``, UE8M0 ``scales [N/128][K/128]``
    -> bf16 bits ``[M][N]``."""
    x_bits = _c(x_bits, np.uint16)
    M, K = x_bits.shape
    N = w_codes.shape[0]
    assert w_codes.shape == (N, K) and w_scales.shape == (N // 128, K // 128)
    y = np.empty((M, N), np.uint16)
    lib().oracle_fp8_block_gemm(M, N, K, _p(x_bits), _p(_c(w_codes, np.uint8)), _p(_c(w_scales, np.uint8)),
                                _p(y))
    return y


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_threads(n: int) -> None:
    lib().oracle_set_threads(n)
