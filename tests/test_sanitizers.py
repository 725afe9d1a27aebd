"""AddressSanitizer + UndefinedBehaviorSanitizer runs on the CPU.

* The oracle: ``oracle/moe_oracle.c`` with the driver ``oracle/sanitize_main.c``
  (every oracle function once, small shapes, exact-size buffers), built with
  gcc; leaks are checked too.
* The library's host code: every HIP source of the package built with the
  sanitizers on its host pass only (the device code is built as usual and
  never runs here), linked with ``tests/host_checks.c``, which drives the
  argument checks of every entry point in ``include/moe_w4a16.h`` with calls
  that must all be rejected before anything is enqueued.

Both build into a temporary directory; nothing is written into the tree."""
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


@pytest.fixture
def tmpdir_clean():
    d = tempfile.mkdtemp(prefix="moe_san_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_clean_under_asan_ubsan(tmpdir_clean):
    exe = os.path.join(tmpdir_clean, "oracle_san")
    rc, out = _run(["gcc", "-O1", "-std=c11", "-ffp-contract=off", "-fopenmp"] + SAN +
                   ["-fsanitize=float-cast-overflow",
                    os.path.join(ROOT, "oracle", "sanitize_main.c"), os.path.join(ROOT, "oracle", "moe_oracle.c"),
                    "-o", exe, "-lm"])
    assert rc == 0, out
    rc, out = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="2"), timeout=300)
    print(out)
    assert rc == 0 and "runtime error" not in out and "ERROR:" not in out, out


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("gcc") is None, reason="hipcc or gcc not found")
def test_host_checks_clean_under_asan_ubsan(tmpdir_clean):
    from w4a16_routed_expert_moe_amd import build as b
    host_san = []
    for flag in ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]:
        host_san += ["-Xarch_host", flag]   # the sanitizers on the host pass only

    def compile_one(src):
        obj = os.path.join(tmpdir_clean, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops"] + host_san + ["-I", os.path.join(ROOT, "include"), "-I", b.CSRC,
                                                           "-c", os.path.join(b.CSRC, src), "-o", obj]
        rc, out = _run(cmd)
        assert rc == 0, out
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(b.SOURCES))) as ex:
        objs = list(ex.map(compile_one, b.SOURCES))
    drv = os.path.join(tmpdir_clean, "host_checks.o")
    rc, out = _run(["gcc", "-O1", "-std=c11", "-Wall"] + SAN + ["-I", os.path.join(ROOT, "include"), "-c",
                                                               os.path.join(ROOT, "tests", "host_checks.c"),
                                                               "-o", drv])
    assert rc == 0, out
    exe = os.path.join(tmpdir_clean, "host_checks")
    rc, out = _run([HIPCC, "--offload-arch=gfx950"] + host_san[:4] + ["-o", exe, drv] + objs)
    assert rc == 0, out
    rc, out = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"), timeout=300)
    print(out)
    assert rc == 0 and "runtime error" not in out and "ERROR:" not in out, out
