"""The LDS-tiled GEMMs' k step, checked on the compiled code (CPU only).

Each step of ``k_w4a16_tiled`` / ``k_mxfp4_tiled`` issues the next k group's
activation loads into LDS and then, last, the weight loads of the group after
it.  The next step waits until at most that many weight loads are outstanding
and then reads the LDS stage that every wave of the workgroup filled.  If the
compiler scheduled a load into LDS after the weight loads, that wait would not
cover it and another wave could read the stage before the load lands.  This
test compiles moe_gemm_tiled.hip with the library's flags to gfx950 assembly
and checks, in every tiled kernel, that no ``global_load_lds`` follows a weight
load before the next workgroup barrier."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _functions(asm_lines):
    """{name: [lines]} of the tiled kernels' bodies."""
    out, fn = {}, None
    for line in asm_lines:
        m = re.match(r"^(_Z\S+):", line)
        if m:
            fn = m.group(1) if "_tiled" in m.group(1) else None
            if fn:
                out[fn] = []
            continue
        if fn is not None:
            if line.startswith(".Lfunc_end"):
                fn = None
            else:
                out[fn].append(line.split(";")[0].strip())
    return out


def _is_weight_load(op):
    # the step's weight operands: INT4 / FP4 code words and FP4 scale bytes
    return op.startswith(("global_load_dwordx4", "global_load_ubyte"))


def misplaced_lds_loads(asm_lines):
    """(function, instruction) of every load into LDS that some path reaches
    after a weight load with no s_barrier in between, in the tiled kernels: a
    may-analysis over the basic blocks (the compiler lays a loop's blocks out
    in any order, so the text alone does not show what precedes what)."""
    bad = []
    for fn, body in _functions(asm_lines).items():
        blocks, labels, cur = [], {}, []
        for ins in body:
            if not ins:
                continue
            m = re.match(r"^(\.LBB\w+):", ins)
            if m:
                if cur:
                    blocks.append(cur)
                cur = []
                labels[m.group(1)] = len(blocks)
                continue
            if ins.startswith("."):
                continue
            cur.append(ins)
            if ins.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
                blocks.append(cur)
                cur = []
        if cur:
            blocks.append(cur)
        succ = []
        for i, blk in enumerate(blocks):
            last = blk[-1] if blk else ""
            op = last.split()[0] if last else ""
            nxt = []
            if op == "s_branch" or op.startswith("s_cbranch"):
                nxt.append(labels[last.split()[1]])
            if op not in ("s_branch", "s_endpgm", "s_setpc_b64") and i + 1 < len(blocks):
                nxt.append(i + 1)
            succ.append(nxt)

        def transfer(blk, state, report):
            for ins in blk:
                op = ins.split()[0]
                if op.startswith("s_barrier"):
                    state = False
                elif op.startswith("global_load_lds"):
                    if state and report:
                        bad.append((fn, ins))
                elif _is_weight_load(op):
                    state = True
            return state

        state_in = [False] * len(blocks)
        work = list(range(len(blocks)))
        while work:
            i = work.pop()
            out = transfer(blocks[i], state_in[i], False)
            for j in succ[i]:
                if out and not state_in[j]:
                    state_in[j] = True
                    work.append(j)
        for i, blk in enumerate(blocks):
            transfer(blk, state_in[i], True)
    return bad


def test_the_checker_flags_a_misplaced_load():
    # a loop whose body is laid out before its header: the barrier at the
    # header covers the body's loads; a load into LDS after the weights
    # (second case) is flagged
    def loop(tail):
        return ["_ZN3moe1k_w4a16_tiledE:", "s_branch .LBB0_2",
                ".LBB0_1:"] + tail + [
                ".LBB0_2:", "s_waitcnt vmcnt(1)", "s_barrier", "ds_read_b128 v[0:3], v4",
                "s_cbranch_scc1 .LBB0_1", "s_endpgm", ".Lfunc_end0:"]
    assert misplaced_lds_loads(loop(["global_load_lds_dwordx4 v[8:9], off",
                                     "global_load_dwordx4 v[2:5], v[6:7], off"])) == []
    assert misplaced_lds_loads(loop(["global_load_dwordx4 v[2:5], v[6:7], off",
                                     "global_load_lds_dwordx4 v[8:9], off"])) == [
        ("_ZN3moe1k_w4a16_tiledE", "global_load_lds_dwordx4 v[8:9], off")]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_no_load_into_lds_after_the_weight_loads_of_a_step():
    from w4a16_routed_expert_moe_amd import build as b
    d = tempfile.mkdtemp(prefix="moe_asm_")
    try:
        out = os.path.join(d, "tiled.s")
        flags = [f for f in b.FLAGS if f != "-fPIC"] + b.EXTRA.get("moe_gemm_tiled.hip", [])
        r = subprocess.run([HIPCC] + flags + ["--cuda-device-only", "-S", "-o", out,
                                              os.path.join(b.CSRC, "moe_gemm_tiled.hip")],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        lines = open(out).read().splitlines()
    finally:
        shutil.rmtree(d, ignore_errors=True)
    kernels = {m.group(1) for m in (re.match(r"^(_Z\S*_tiled\S*):", x) for x in lines) if m}
    assert len(kernels) >= 8, kernels  # every INT4 and FP4 instance was compiled
    bad = misplaced_lds_loads(lines)
    assert not bad, "loads into LDS after a step's weight loads: %s" % bad[:5]
