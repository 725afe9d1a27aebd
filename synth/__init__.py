"""Seeded synthetic inputs for the W4A16 routed-expert MoE layer.

This module only draws inputs. It holds none of the layer's arithmetic
(no routing, no dequantisation, no matmul) and is the one module that both
the CPU oracle side (``oracle/``, ``tests/``) and the HIP side (``bench.py``,
GPU tests) import.

Workload recipe (shapes from the model card "canada-quant/DeepSeek-V4-Flash-W4A16-FP8-MTP",
section "Architecture & precision": hidden 4096, 256 routed experts, top-6,
routed experts stored as INT4 with group_size=128, symmetric):

* activations ``x``: N(0, 1) drawn in fp32, rounded to bf16 (RNE);
* router weight ``W_r``: N(0, 0.02) (0.02 is the standard deviation), bf16;
* gate bias ``b``: U(-0.1, 0.1) in fp32 (the card keeps ``ffn.gate.bias`` in FP32);
* INT4 codes: uniform on [-8, 7], from a counter-based SplitMix64 hash so any
  tensor of any layer can be regenerated on its own (host here, device in
  the library's ``moe_gen_*`` entry points, which implement the same
  published generator independently);
* fp16 group scales: U(0.005, 0.02) built from the same hash;
* FP4 weights (the release's own expert format): the same uniform nibbles
  read as E2M1 codes, with UE8M0 scales (one per 32 elements along K)
  E = 120 + (h >> 62), i.e. 2^-7 .. 2^-4, so the weights have the INT4
  workload's magnitude.

SplitMix64 is the generator of Steele, Lea & Flood, "Fast splittable
pseudorandom number generators" (OOPSLA 2014): state advances by the golden
gamma 0x9E3779B97F4A7C15 and each state is passed through the two
xor-shift-multiply rounds (0xBF58476D1CE4E5B9, 0x94D049BB133111EB, shifts 30,
27, 31).  Output ``i`` of the stream seeded with ``s`` is ``mix(s + (i+1)*gamma)``.
"""
from __future__ import annotations

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

# Tensor kinds of one expert group, used to derive per-tensor stream seeds.
KIND_W13 = 0      # gate/up INT4 codes, canonical [2I][H/2] bytes
KIND_W2 = 1       # down INT4 codes, canonical [H][I/2] bytes
KIND_S13 = 2      # gate/up fp16 scales [2I][H/128]
KIND_S2 = 3       # down fp16 scales [H][I/128]
GROUPS_STRIDE = 512  # fixed stride for the group index inside a tensor id (>= any G)


# ---------------------------------------------------------------------------
# SplitMix64 (counter form)
# ---------------------------------------------------------------------------
def splitmix64_py(seed: int, index: int) -> int:
    """Output ``index`` (0-based) of the SplitMix64 stream seeded with ``seed``
    (plain Python integers; the scalar reference used to check the vector form)."""
    z = (seed + (index + 1) * GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * _M1) & MASK64
    z = ((z ^ (z >> 27)) * _M2) & MASK64
    return z ^ (z >> 31)


def _mix_u64(z: np.ndarray) -> np.ndarray:
    z = z.copy()
    z ^= z >> np.uint64(30)
    z *= np.uint64(_M1)
    z ^= z >> np.uint64(27)
    z *= np.uint64(_M2)
    z ^= z >> np.uint64(31)
    return z


def splitmix64_block(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs ``start .. start+count-1`` of the stream seeded with ``seed`` (uint64)."""
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & MASK64) + idx * np.uint64(GAMMA)
        return _mix_u64(z)


def tensor_seed(seed: int, layer: int, group: int, kind: int) -> int:
    """Stream seed of one weight tensor: output number ``tid`` of the run's stream,
    ``tid = ((layer * 512) + group) * 4 + kind``."""
    tid = ((layer * GROUPS_STRIDE) + group) * 4 + kind
    return splitmix64_py(seed, tid)


def int4_codes(seed: int, layer: int, group: int, kind: int, n: int, k: int) -> np.ndarray:
    """Canonical packed INT4 codes ``[n][k/2]`` (uint8) for one projection.

    Word ``i`` of the stream is the little-endian 8 bytes ``8i .. 8i+7`` of the
    row-major byte array; byte ``c`` of row ``r`` holds element ``2c`` in its low
    nibble and ``2c+1`` in its high nibble, each a two's-complement code in
    [-8, 7].  Every byte pattern is equally likely, so codes are uniform.
    """
    assert k % 16 == 0
    nbytes = n * k // 2
    words = splitmix64_block(tensor_seed(seed, layer, group, kind), 0, nbytes // 8)
    return words.astype("<u8").view(np.uint8).reshape(n, k // 2)


def fp16_scales(seed: int, layer: int, group: int, kind: int, n: int, k: int) -> np.ndarray:
    """fp16 scales ``[n][k/128]``: ``u = (h >> 40) * 2^-24``, ``s = fmaf(0.015, u, 0.005)``
    rounded to fp16 (RNE).  The fused multiply-add is evaluated exactly in fp64
    (both products and the sum fit in 53 bits) and rounded once to fp32."""
    assert k % 128 == 0
    cnt = n * (k // 128)
    h = splitmix64_block(tensor_seed(seed, layer, group, kind), 0, cnt)
    u = (h >> np.uint64(40)).astype(np.float64) * 2.0 ** -24
    s32 = (np.float64(np.float32(0.015)) * u + np.float64(np.float32(0.005))).astype(np.float32)
    return s32.astype(np.float16).reshape(n, k // 128)


def ue8m0_scales(seed: int, layer: int, group: int, kind: int, n: int, k: int) -> np.ndarray:
    """UE8M0 scale bytes ``[n][k/32]``: ``E = 120 + (h >> 62)``."""
    assert k % 32 == 0
    cnt = n * (k // 32)
    h = splitmix64_block(tensor_seed(seed, layer, group, kind), 0, cnt)
    return (np.uint64(120) + (h >> np.uint64(62))).astype(np.uint8).reshape(n, k // 32)


def fp4_expert_weights(seed: int, layer: int, group: int, hidden: int, inter: int):
    """The four tensors of one expert group with FP4 weights: ``w13 [2I][H/2] u8``
    and ``w2 [H][I/2] u8`` (E2M1 codes, packed like the INT4 codes),
    ``s13 [2I][H/32] u8`` and ``s2 [H][I/32] u8`` (UE8M0)."""
    w13 = int4_codes(seed, layer, group, KIND_W13, 2 * inter, hidden)
    w2 = int4_codes(seed, layer, group, KIND_W2, hidden, inter)
    s13 = ue8m0_scales(seed, layer, group, KIND_S13, 2 * inter, hidden)
    s2 = ue8m0_scales(seed, layer, group, KIND_S2, hidden, inter)
    return w13, s13, w2, s2


def stacked_fp4_expert_weights(seed: int, layer: int, n_groups: int, hidden: int, inter: int):
    """``fp4_expert_weights`` for groups ``0..n_groups-1`` stacked along a leading axis."""
    parts = [fp4_expert_weights(seed, layer, g, hidden, inter) for g in range(n_groups)]
    return tuple(np.stack([p[i] for p in parts]) for i in range(4))


def expert_weights(seed: int, layer: int, group: int, hidden: int, inter: int):
    """All four tensors of one expert group in canonical layout:
    ``w13 [2I][H/2] u8`` (rows ``[0,I)`` gate, ``[I,2I)`` up), ``s13 [2I][H/128] f16``,
    ``w2 [H][I/2] u8``, ``s2 [H][I/128] f16``."""
    w13 = int4_codes(seed, layer, group, KIND_W13, 2 * inter, hidden)
    w2 = int4_codes(seed, layer, group, KIND_W2, hidden, inter)
    s13 = fp16_scales(seed, layer, group, KIND_S13, 2 * inter, hidden)
    s2 = fp16_scales(seed, layer, group, KIND_S2, hidden, inter)
    return w13, s13, w2, s2


def stacked_expert_weights(seed: int, layer: int, n_groups: int, hidden: int, inter: int):
    """The four tensors for groups ``0..n_groups-1`` stacked along a leading axis."""
    parts = [expert_weights(seed, layer, g, hidden, inter) for g in range(n_groups)]
    return tuple(np.stack([p[i] for p in parts]) for i in range(4))


# ---------------------------------------------------------------------------
# bf16 storage helpers (storage conversion only)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(np.asarray(a, dtype=np.float32))
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# Activations, router weight and bias
# ---------------------------------------------------------------------------
def _rng(seed: int, stream: int, layer: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, stream, layer]))


STREAM_X, STREAM_WR, STREAM_BIAS, STREAM_ZIPF, STREAM_UNIFORM = 1, 2, 3, 4, 5
FP8_GROUP = 511  # tensor ids of the FP8_BLOCK projection: group slot 511 (no expert has it),
                 # kind 0 codes, kind 1 scales


def fp8_block_weights(seed: int, layer: int, N: int, K: int):
    """An FP8_BLOCK projection weight: e4m3 codes ``[N][K]`` (u8) and UE8M0 scales
    ``[N/128][K/128]`` (u8).  Each code byte is a SplitMix64 output byte b taken
    as sign = bit 7, exponent field 5 + ((b >> 3) & 3), mantissa = b & 7 (never NaN;
    magnitudes 0.25 .. 3.75); each scale is E = 120 + (h >> 62) (2^-7 .. 2^-4), so
    the weights have the magnitude of the expert weights."""
    assert N % 128 == 0 and K % 128 == 0
    raw = splitmix64_block(tensor_seed(seed, layer, FP8_GROUP, 0), 0, N * K // 8).view(np.uint8)
    codes = (raw & 0x80) | ((5 + ((raw >> 3) & 3)) << 3) | (raw & 7)
    h = splitmix64_block(tensor_seed(seed, layer, FP8_GROUP, 1), 0, (N // 128) * (K // 128))
    scales = (120 + (h >> np.uint64(62))).astype(np.uint8)
    return codes.astype(np.uint8).reshape(N, K), scales.reshape(N // 128, K // 128)


def make_x(T: int, H: int, seed: int = 0) -> np.ndarray:
    """Activations x ~ N(0,1), bf16 bits ``[T][H]``."""
    return f32_to_bf16_bits(_rng(seed, STREAM_X).standard_normal((T, H), dtype=np.float32))


def make_router(E: int, H: int, seed: int = 0, layer: int = 0) -> np.ndarray:
    """Router weight W_r ~ N(0, 0.02), bf16 bits ``[E][H]``."""
    w = _rng(seed, STREAM_WR, layer).standard_normal((E, H), dtype=np.float32) * np.float32(0.02)
    return f32_to_bf16_bits(w)


def make_bias(E: int, seed: int = 0, layer: int = 0) -> np.ndarray:
    """Gate bias b ~ U(-0.1, 0.1), fp32 ``[E]``."""
    return _rng(seed, STREAM_BIAS, layer).uniform(-0.1, 0.1, E).astype(np.float32)


def make_zipf_router(T: int, H: int, E: int, seed: int = 0, s: float = 1.1,
                     logit_std: float = 1.3, layer: int = 0):
    """Activations and a router weight whose logits give Zipf(s)-skewed expert load.

    Construction: expert popularity ``p_e ~ (pi(e)+1)^-s`` for a seeded permutation
    ``pi``; per-token target logits ``L = log p + Gumbel(0,1)`` (the Gumbel-top-k
    trick of Kool, van Hoof & Welling 2019 makes the top-k of ``L`` a draw without
    replacement from ``p``); each row standardised to ``logit_std``; then
    ``W_r^T = X^T (X X^T)^{-1} L`` in fp64 (minimum-norm exact fit to the bf16
    activations) rounded to bf16.  Returns ``(x_bits [T][H], wr_bits [E][H])``.
    Every ``layer`` shares the same activations and draws its own popularity
    permutation and noise.
    """
    rng = _rng(seed, STREAM_ZIPF, layer)
    x_bits = make_x(T, H, seed)
    X = bf16_bits_to_f32(x_bits).astype(np.float64)
    perm = rng.permutation(E)
    p = (perm + 1.0) ** (-s)
    p /= p.sum()
    L = np.log(p)[None, :] + rng.gumbel(size=(T, E))
    L = (L - L.mean(axis=1, keepdims=True)) / L.std(axis=1, keepdims=True) * logit_std
    WrT = X.T @ np.linalg.solve(X @ X.T, L)
    return x_bits, f32_to_bf16_bits(WrT.T.astype(np.float32))


def make_uniform_x(T: int, H: int, wr_bits: np.ndarray, bias: np.ndarray, seed: int = 0,
                   layer: int = 0, logit_std: float = 1.28, clip: float = 2.1) -> np.ndarray:
    """Activations whose routing keys are i.i.d. across experts: uniform routing.

    With the gate bias in the keys (score + b_e), i.i.d. Gaussian activations
    favour the experts with the larger biases so strongly that at 8192 tokens
    about 30 of 256 experts are never chosen and the loads run from a few rows
    to several hundred.  Here each token's keys are drawn i.i.d. instead, so its
    top-k is a uniformly random k-subset of the experts, and the activations are
    made to produce them:

    * target keys ``k_te = sigmoid(Y_te)``, ``Y_te ~ N(0, logit_std^2)`` clipped
      to ``[-clip, clip]`` (keys in (0.109, 0.891), so ``k - b`` stays in (0, 1));
    * target scores ``s_te = k_te - b_e`` and target logits ``L_te = logit(s_te)``;
    * ``x_t = z_t + W^+ (L_t - W z_t)`` with ``z_t`` the standard-normal draw of
      :func:`make_x`, ``W`` the bf16 router weight in fp64 and
      ``W^+ = W^T (W W^T)^-1``: the component of ``z_t`` in the span of the router
      rows is replaced by the one that gives ``W x_t = L_t`` exactly.  The other
      ``H - E`` directions keep their N(0,1) draw and the replaced ones carry about
      the same variance (``logit_std^2`` is the variance of ``W z``), so ``x`` stays
      close to N(0,1); rounding to bf16 moves the logits by a few 1e-3.

    Returns ``x_bits [T][H]``.
    """
    rng = _rng(seed, STREAM_UNIFORM, layer)
    W = bf16_bits_to_f32(wr_bits).astype(np.float64)
    Z = _rng(seed, STREAM_X).standard_normal((T, H), dtype=np.float32).astype(np.float64)
    Y = np.clip(rng.standard_normal((T, W.shape[0])) * logit_std, -clip, clip)
    S = 1.0 / (1.0 + np.exp(-Y)) - bias.astype(np.float64)[None, :]
    L = np.log(S / (1.0 - S))
    X = Z + (L - Z @ W.T) @ np.linalg.solve(W @ W.T, W)
    return f32_to_bf16_bits(X.astype(np.float32))


# ---------------------------------------------------------------------------
# Workload table
# ---------------------------------------------------------------------------
WORKLOADS = {
    # name: (T, H, E, k, n_shared, I, routing, layers)
    "tiny": dict(T=8, H=512, E=16, k=2, n_shared=1, I=256, routing="iid", layers=1),
    "decode1": dict(T=1, H=4096, E=256, k=6, n_shared=1, I=2048, routing="iid", layers=1),
    "decode64": dict(T=64, H=4096, E=256, k=6, n_shared=1, I=2048, routing="zipf", layers=1),
    "prefill8k": dict(T=8192, H=4096, E=256, k=6, n_shared=1, I=2048, routing="uniform", layers=1),
    "stack43": dict(T=2048, H=4096, E=256, k=6, n_shared=1, I=2048, routing="iid", layers=43),
}


def make_router_inputs(name: str, seed: int = 0, layer: int = 0, T: int | None = None):
    """``(x_bits, wr_bits, bias)`` for a workload (``T`` overrides the token count)."""
    w = WORKLOADS[name]
    T = w["T"] if T is None else T
    bias = make_bias(w["E"], seed, layer)
    if w["routing"] == "zipf":
        x, wr = make_zipf_router(T, w["H"], w["E"], seed, layer=layer)
    elif w["routing"] == "uniform":
        wr = make_router(w["E"], w["H"], seed, layer)
        x = make_uniform_x(T, w["H"], wr, bias, seed, layer)
    else:
        x = make_x(T, w["H"], seed)
        wr = make_router(w["E"], w["H"], seed, layer)
    return x, wr, bias
