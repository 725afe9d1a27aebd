"""The C-ABI library loads, exports every symbol its header declares, and its
host-side argument checks return the documented status before anything is
enqueued (no kernel is launched here, so no GPU is needed)."""
import ctypes
import os
import re

import pytest

import w4a16_routed_expert_moe_amd as moe
from w4a16_routed_expert_moe_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, UNSUP, ALIGN, DEVICE, WORKSPACE = 0, 1, 2, 3, 4, 6, 7


def _header_functions():
    with open(os.path.join(ROOT, "include", "moe_w4a16.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char \*|int32_t|size_t)\s*\**\s*(moe_\w+)\s*\(",
                                 text, re.M)))


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    names = _header_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    assert _lib.moe_abi_version() == 10 == _lib.ABI_VERSION
    assert _lib.moe_status_str(2) == "size outside the supported limits"
    assert _lib.moe_status_str(99) == "unknown status"


def _desc(**kw):
    base = dict(hidden=4096, inter=2048, n_routed=256, top_k=6, n_shared=1, routed_scale=1.0)
    base.update(kw)
    return moe.MoeLayerDesc.make(**base)


P = ctypes.c_void_p
FAKE = P(0x1000)          # never dereferenced: every call below fails validation first
FAKE_ODD = P(0x1002)

# The calls with placeholder pointers must never reach a kernel launch; as a
# second guard they only run where no GPU is visible.
import torch  # noqa: E402

no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="placeholder-pointer checks run without a GPU")


@no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(hidden=4000), SHAPE), (dict(hidden=256), SHAPE), (dict(inter=100), SHAPE),
    (dict(n_routed=300), SHAPE), (dict(top_k=9), SHAPE), (dict(n_routed=4, top_k=5), SHAPE),
    (dict(n_shared=2), SHAPE), (dict(routed_scale=float("nan")), SHAPE),
])
def test_descriptor_limits(kw, status):
    L = _lib.lib()
    assert L.moe_permute(ctypes.byref(_desc(**kw)), 4, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == status
    assert L.moe_combine(ctypes.byref(_desc(**kw)), 4, FAKE, FAKE, FAKE, FAKE, None) == status


@no_gpu
def test_group_size_other_than_128_is_unsupported():
    d = _desc()
    d.group_size = 64
    assert _lib.lib().moe_combine(ctypes.byref(d), 4, FAKE, FAKE, FAKE, FAKE, None) == UNSUP


@no_gpu
def test_null_align_and_token_checks():
    L = _lib.lib()
    d = ctypes.byref(_desc())
    assert L.moe_route(d, 4, None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == NULL
    assert L.moe_route(d, 4, FAKE_ODD, FAKE, FAKE, FAKE, FAKE, FAKE, None) == ALIGN
    assert L.moe_route(d, -1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert L.moe_route(d, (1 << 20) + 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert L.moe_route(d, 0, None, None, None, None, None, None, None) == OK
    assert L.moe_permute(d, 4, FAKE, None, FAKE, FAKE, None, 0, None) == NULL
    assert L.moe_combine(d, 4, FAKE_ODD, FAKE, FAKE, FAKE, None) == ALIGN
    g = L.moe_w4a16_grouped_gemm
    assert g(d, 4, FAKE, None, 0, None, 4096, 2048, FAKE, FAKE, FAKE, 7, FAKE, None) == UNSUP
    assert g(d, 4, FAKE, None, 0, None, 4000, 2048, FAKE, FAKE, FAKE, 0, FAKE, None) == SHAPE
    assert g(d, 4, FAKE, None, 0, None, 4096, 2000, FAKE, FAKE, FAKE, 0, FAKE, None) == SHAPE
    assert g(d, 4, None, None, 0, None, 4096, 2048, FAKE, FAKE, FAKE, 0, FAKE, None) == NULL
    assert g(d, 4, FAKE_ODD, None, 0, None, 4096, 2048, FAKE, FAKE, FAKE, 0, FAKE, None) == ALIGN
    assert g(d, 4, FAKE, None, 0, P(0x1002), 4096, 2048, FAKE, FAKE, FAKE, 0, FAKE, None) == ALIGN
    assert L.moe_row_sums(4, 100, FAKE, FAKE, None) == SHAPE
    assert L.moe_row_sums(-1, 128, FAKE, FAKE, None) == SHAPE
    assert L.moe_row_sums(4, 128, None, FAKE, None) == NULL
    assert L.moe_row_sums(4, 128, FAKE_ODD, FAKE, None) == ALIGN
    assert L.moe_row_sums(0, 128, None, None, None) == OK
    dc = L.moe_w4a16_down_combine
    assert dc(d, 5, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == UNSUP       # T > 4
    assert dc(ctypes.byref(_desc(inter=384)), 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == UNSUP
    assert dc(d, 1, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == NULL
    assert dc(d, 1, FAKE_ODD, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == ALIGN
    assert dc(d, 0, None, None, None, None, None, None, None, None) == OK
    dt = L.moe_w4a16_decode_token
    args = [FAKE] * 16
    assert dt(ctypes.byref(_desc(hidden=1024)), *args, None) == UNSUP
    assert dt(ctypes.byref(_desc(inter=4096)), *args, None) == UNSUP        # 7 * 32 down blocks > 112
    assert dt(d, None, *args[1:], None) == NULL
    assert dt(d, *args[:15], None, None) == NULL                             # workspace
    assert dt(d, FAKE_ODD, *args[1:], None) == ALIGN
    assert dt(d, *args[:15], P(0x1008), None) == ALIGN                       # workspace 16-byte aligned
    assert dt(d, *args, None) == DEVICE                                       # no GPU here: nothing launched
    df = L.moe_mxfp4_decode_token                                            # the same checks, FP4 weights
    assert df(ctypes.byref(_desc(hidden=1024)), *args, None) == UNSUP
    assert df(d, *args[:5], None, *args[6:], None) == NULL                   # w13_scales
    assert df(d, *args[:5], P(0x1004), *args[6:], None) == ALIGN             # w13_scales 16-byte aligned
    assert df(d, *args, None) == DEVICE
    assert L.moe_w4a16_decode_token_supported(d) == DEVICE
    assert L.moe_w4a16_decode_token_supported(ctypes.byref(_desc(hidden=512, inter=256, n_routed=16,
                                                                 top_k=2))) == UNSUP
    assert L.moe_w4a16_prepack(1, 4096, 2000, FAKE, FAKE, None) == SHAPE
    assert L.moe_w4a16_prepack(1, 4096, 2048, FAKE, FAKE, None) == SHAPE  # overlapping buffers
    assert L.moe_gen_int4_codes(0, 0, 0, 1, 4, 16, 128, FAKE, None) == SHAPE
    assert L.moe_gen_fp16_scales(0, 0, 510, 3, 0, 16, 128, FAKE, None) == SHAPE


def test_decode_workspace_size_matches_header():
    with open(os.path.join(ROOT, "include", "moe_w4a16.h")) as f:
        m = re.search(r"#define MOE_DECODE_WORKSPACE_BYTES (\d+)", f.read())
    assert int(m.group(1)) == _lib.MOE_DECODE_WORKSPACE_BYTES == moe.MOE_DECODE_WORKSPACE_BYTES


def test_binding_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        _lib.moe_combine(_desc(), 1, torch.zeros(7 * 4096, dtype=torch.bfloat16),
                         torch.zeros(7, dtype=torch.int32), torch.zeros(6), torch.zeros(4096, dtype=torch.bfloat16))


@no_gpu
def test_mxfp4_argument_checks():
    L = _lib.lib()
    d = ctypes.byref(_desc())
    gemm = lambda T, a, N, K, s, act: L.moe_mxfp4_grouped_gemm(d, T, a, None, 0, N, K, FAKE, s, FAKE, act,
                                                               FAKE, None)
    assert gemm(4, FAKE, 192, 2048, FAKE, 0) == SHAPE        # N not a multiple of 128
    assert gemm(4, FAKE, 4096, 8192, FAKE, 0) == SHAPE       # K above 4096
    assert gemm(4, FAKE, 4096, 2048, FAKE, 7) == UNSUP       # unknown activation
    assert gemm(4, FAKE, 4096, 2048, None, 0) == NULL
    assert gemm(4, FAKE_ODD, 4096, 2048, FAKE, 0) == ALIGN
    assert gemm(4, FAKE, 4096, 2048, P(0x1008), 0) == ALIGN   # scales 16-byte aligned
    assert gemm(0, None, 4096, 2048, None, 0) == OK          # T = 0: nothing enqueued
    assert L.moe_mxfp4_prepack(4, 8, 128, FAKE, FAKE, None) == SHAPE
    assert L.moe_mxfp4_prepack(4, 16, 128, None, FAKE, None) == NULL
    assert L.moe_mxfp4_prepack(0, 16, 128, None, None, None) == OK
    assert L.moe_gen_ue8m0_scales(0, 0, 0, 1, 2, 16, 48, FAKE, None) == SHAPE   # K % 32
    assert L.moe_gen_ue8m0_scales(0, 0, 0, 1, 2, 16, 64, None, None) == NULL


def test_workspace_bytes():
    # a 256-byte header, plus 1280 bytes per 1024-token chunk past the first
    L = _lib.lib()
    d = ctypes.byref(_desc())
    assert L.moe_workspace_bytes(d, 0) == 256
    assert L.moe_workspace_bytes(d, 1) == 256
    assert L.moe_workspace_bytes(d, 1024) == 256
    assert L.moe_workspace_bytes(d, 1025) == 256 + 2 * 1280
    assert L.moe_workspace_bytes(d, 8192) == 256 + 8 * 1280
    assert L.moe_workspace_bytes(d, 1 << 20) == 256 + 1024 * 1280
    assert L.moe_workspace_bytes(d, -1) == 0
    assert L.moe_workspace_bytes(d, (1 << 20) + 1) == 0
    assert L.moe_workspace_bytes(ctypes.byref(_desc(hidden=4000)), 8) == 0
    assert L.moe_workspace_bytes(None, 8) == 0
    assert _lib.moe_workspace_bytes(_desc(), 8192) == 256 + 8 * 1280


@no_gpu
def test_workspace_checks():
    L = _lib.lib()
    d = ctypes.byref(_desc())
    need = L.moe_workspace_bytes(d, 2000)
    p = L.moe_permute
    assert p(d, 2000, FAKE, FAKE, FAKE, FAKE, None, need, None) == NULL          # two chunks need it
    assert p(d, 2000, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == WORKSPACE
    assert p(d, 2000, FAKE, FAKE, FAKE, FAKE, P(0x1008), need, None) == ALIGN
    rp = L.moe_route_permute
    args = [FAKE] * 9
    assert rp(d, 3, *args, None, 256, None) == NULL                            # the counter lives there
    assert rp(d, 3, *args, FAKE, 255, None) == WORKSPACE
    assert rp(d, 3, *args, P(0x1004), 256, None) == ALIGN
    assert rp(d, 0, *([None] * 9), None, 0, None) == OK


def test_package_wraps_every_entry_point():
    # each exported C function has a binding of the same name on the package
    # (the version and status-string helpers are wrapped in _lib only)
    missing = [n for n in _lib.EXPORTS
               if n not in ("moe_status_str", "moe_abi_version") and not hasattr(moe, n)]
    assert not missing, missing
