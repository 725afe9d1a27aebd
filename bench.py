"""Benchmark of the W4A16 routed-expert MoE layer on one MI355X.

A step is one full forward pass of the layer (route, permute, gate/up GEMM
with SwiGLU, down GEMM, combine) over one batch of synthetic tokens.  The
weights of ``--layers`` independent layers stay resident in HBM and step i
runs layer i mod L, so consecutive steps read different expert weights and
the 256 MB Infinity Cache cannot serve them (a decode step reads ~93 MB).

Timing: W eager warm-up steps, then K steps captured in one HIP graph,
replayed once untimed and once between events (synchronised on both sides).
The dominant kernel (the gate/up grouped GEMM) is also timed on its own:
nk back-to-back launches over the same layer rotation, captured in a graph
and bracketed by HIP events on the stream it is launched on; the average
launch duration is priced against the kernel's roofline.  The CPU oracle is timed on a
bounded sample of the same workload for the ``cpu_baseline`` field.

``--format fp4`` runs the same layer with FP4 expert weights (E2M1 codes, one
UE8M0 scale per 32 along K; both GEMMs through moe_mxfp4_grouped_gemm).

One run measures the whole metric: the headline workload (``--workload``,
decode1 by default: one token, the bs=1 decode step) gives the top-level
fields, and every other workload of the metric (decode64, prefill8k and the
43-layer stack at 2048 tokens) gets a block under ``configs`` with its own
ms/step, tokens/s, ``roofline`` (dominant kernel) and ``layer_roofline``
(the whole layer step against its algorithmic bytes or FLOP).  The workloads
share one resident set of expert weights (layer li's experts do not depend on
the workload).  ``--only`` runs the headline workload alone.

Prints one JSON line (progress lines go to stderr).  ``--gpus N`` with N > 1
is refused: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s on 1 MI355X (bs=1,64,2048; 8192 prefill) + % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, TFLOP/s

DEFAULT_LAYERS = {"decode1": 8, "decode64": 4, "prefill8k": 2, "stack43": 43}
DEFAULT_STEPS = {"decode1": 200, "decode64": 100, "prefill8k": 20, "stack43": 86}
TILED_MIN_TOKENS = 384  # the grouped GEMM takes its LDS-tiled kernel from here on
CSRC = os.path.join(ROOT, "w4a16_routed_expert_moe_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
FP8_PROJ = "proj8192x4096x4096"  # the FP8_BLOCK projection GEMM: M x N x K


def dominant_kernel(T, fmt="int4"):
    """(name, rocprofv3 name prefix, source files) of the kernel priced against
    its roofline at T tokens: the one-launch decode step at one token (the
    whole layer), else the gate/up GEMM (fmt "fp8_block": the projection
    GEMM of e4m3 weights)."""
    common = ["moe_common.h", "moe_gemm_common.h"]
    if fmt == "fp8_block":
        return "k_mx_gemm", "k_mx_gemm<0, 0,", common + ["moe_mx_gemm.hip"]
    if fmt == "w4a8":
        if T == 1:
            return ("k_w4a8_decode_token", "k_w4a8_decode_token<",
                    common + ["moe_route_common.h", "moe_decode.hip"])
        if T < TILED_MIN_TOKENS:  # the quantised activations in bf16 through the FP4 weight stream
            return "k_mxfp4_stream", "k_mxfp4_stream<1,", common + ["moe_gemm.hip"]
        return "k_mx_gemm", "k_mx_gemm<4, 1,", common + ["moe_mx_gemm.hip"]
    if fmt == "fp4":
        if T == 1:
            return ("k_mxfp4_decode_token", "k_mxfp4_decode_token<",
                    common + ["moe_route_common.h", "moe_decode.hip"])
        if T >= TILED_MIN_TOKENS:  # the layer's N (4096) takes the 512-wide FP4 tiles
            return "k_mxfp4_wide", "k_mxfp4_wide<1,", common + ["moe_gemm_fp4wide.hip"]
        return "k_mxfp4_stream", "k_mxfp4_stream<1,", common + ["moe_gemm.hip"]
    if T == 1:
        return "k_decode_token", "k_decode_token<", common + ["moe_route_common.h", "moe_decode.hip"]
    if T >= TILED_MIN_TOKENS:
        return "k_w4a16_tiled", "k_w4a16_tiled<1,", common + ["moe_gemm_tiled.hip"]
    return "k_w4a16_stream", "k_w4a16_stream<1,", common + ["moe_gemm.hip"]


def kernel_source_hash(files):
    import hashlib
    h = hashlib.sha256()
    for f in files + ["../build.py"]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def scale_bytes_per_row(K, fmt):
    """Scale bytes of one weight row of length K: fp16 per 128 (INT4), one UE8M0 byte per 32 (FP4)."""
    return (K // 128) * 2 if fmt == "int4" else K // 32


def traffic_file(kernel, workload):
    return os.path.join(PROFILES, "%s_%s_traffic.json" % (kernel, workload))


def traffic_tag(workload, fmt, kernel):
    """The name a kernel's counter summary goes under: the workload, plus the
    format where the kernel also serves another one (the W4A8 layer's small
    batches run the FP4 weight-stream kernel on its quantised activations)."""
    return workload + "_w4a8" if fmt == "w4a8" and kernel == "k_mxfp4_stream" else workload


def load_traffic(kernel, workload, files):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel's sources changed since it was taken."""
    path = traffic_file(kernel, workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash(files):
        return None
    return int(rec["traffic_bytes_per_launch"])


def ingest_pmc(workload, fetch_csv, write_csv, fmt="int4"):
    """Turn two rocprofv3 --pmc runs of ``bench.py --eager --calib-copy-mib 256``
    (FETCH_SIZE, then WRITE_SIZE) into the traffic summary of the dominant
    kernel: KiB per dispatch, scaled by what each counter reads for the
    calibration copy of known size."""
    import csv
    if workload == FP8_PROJ:
        fmt = "fp8_block"
        kernel, prefix, files = dominant_kernel(0, fmt)
    else:
        T = __import__("synth").WORKLOADS[workload]["T"]
        kernel, prefix, files = dominant_kernel(T, fmt)

    def read(path, counter):
        vals, copies = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"].replace("moe::(anonymous namespace)::", "").replace("void ", "")
            v = float(r["Counter_Value"])
            if name.startswith(prefix):
                vals.append(v)
            elif "copyBuffer" in name:
                copies.append(v)
        if not vals or not copies:
            raise SystemExit("%s: no %s rows for %s or for the calibration copy" % (path, counter, prefix))
        return sum(vals) / len(vals), max(copies), len(vals)

    copy_kib = 256 * 1024
    f_kib, f_copy, n = read(fetch_csv, "FETCH_SIZE")
    w_kib, w_copy, _ = read(write_csv, "WRITE_SIZE")
    f_scale, w_scale = copy_kib / f_copy, copy_kib / w_copy
    rec = {"kernel": kernel, "workload": workload, "dispatches": n,
           "fetch_kib_per_dispatch": round(f_kib, 1), "write_kib_per_dispatch": round(w_kib, 1),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "calibration": "256 MiB device copy: FETCH_SIZE %.0f KiB, WRITE_SIZE %.0f KiB" % (f_copy, w_copy),
           "traffic_bytes_per_launch": int(round((f_kib * f_scale + w_kib * w_scale) * 1024)),
           "source_hash": kernel_source_hash(files),
           "command": ["rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o run -- "
                       "python3 bench.py --workload %s --only --eager --calib-copy-mib 256 --cpu-seconds 0" % workload,
                       "rocprofv3 --pmc WRITE_SIZE (same)",
                       "python3 bench.py --workload %s --ingest-pmc <fetch csv> <write csv>" % workload]}
    if fmt not in ("int4", "fp8_block"):
        rec["command"] = [c.replace("--workload", "--format %s --workload" % fmt) for c in rec["command"]]
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_file(kernel, traffic_tag(workload, fmt, kernel)), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode1", choices=list(DEFAULT_LAYERS) + [FP8_PROJ],
                    help="the headline workload (its figures are the top-level fields); %s runs the "
                         "FP8_BLOCK projection alone (counter runs)" % FP8_PROJ)
    ap.add_argument("--only", action="store_true",
                    help="run the headline workload alone (no per-config block; counter runs)")
    ap.add_argument("--layers", type=int, default=None, help="resident layers in the headline rotation")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--kernel-launches", type=int, default=None,
                    help="launches of the dominant kernel timed with events")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step directly instead of through HIP graphs (for counter runs)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic summary of the dominant kernel from two counter runs")
    ap.add_argument("--format", default="int4", choices=["int4", "fp4", "w4a8"],
                    help="expert weights: INT4 with fp16 scales per 128 (the layer's format), the "
                         "release's FP4 (E2M1, UE8M0 scale per 32), or FP4 with fp8 activations (W4A8)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the oracle baseline sample (0 = skip)")
    return ap.parse_args()


ALL_WORKLOADS = ("decode1", "decode64", "prefill8k", "stack43")


def layer_work(T, H, E, I, counts, fmt):
    """Algorithmic bytes and FLOP of one whole layer step: router rows, x, the
    codes and scales of every touched group (gate/up and down), h and y
    written and read once, out written; 2*T*E*H router FLOP plus 6*H*I per
    permuted row."""
    touched = int((counts > 0).sum())
    R = int(counts.sum())
    wbytes = touched * (3 * I * H // 2 + 2 * I * scale_bytes_per_row(H, fmt) + H * scale_bytes_per_row(I, fmt))
    bytes_ = E * H * 2 + T * H * 2 + wbytes + 2 * R * I * 2 + 2 * R * H * 2 + T * H * 2
    flop = 2.0 * T * E * H + 6.0 * R * I * H
    return bytes_, flop


def roofline(bytes_, flop, seconds, mfma_peak=BF16_PEAK_TFLOPS):
    """Price one measured duration against the roofline of its bound (the
    matrix-core peak of the arithmetic's dtype: bf16, or fp8 for the
    fp8-activation paths)."""
    gbs = bytes_ / seconds / 1e9
    tfs = flop / seconds / 1e12
    ridge = mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    if flop / bytes_ < ridge:
        return dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(gbs / HBM_PEAK_GBS, 4))
    return dict(bound="mfma", achieved=round(tfs, 1), peak=mfma_peak, unit="TFLOP/s",
                frac=round(tfs / mfma_peak, 4))


def run_workload(name, args, experts, steps, warmup, n_layers, fmt):
    """Time one workload over layers 0..n_layers-1 of the resident experts.
    Returns the per-config record (ms/step, tokens/s, rooflines) and the host
    inputs (for the CPU baseline)."""
    import torch

    import synth
    import w4a16_routed_expert_moe_amd as moe

    wl = synth.WORKLOADS[name]
    T, H, E, k, I, ns = wl["T"], wl["H"], wl["E"], wl["k"], wl["I"], wl["n_shared"]
    L, K, W = n_layers, steps, warmup
    w4a8 = fmt == "w4a8"
    # W4A8 below the tiled range: the GEMMs multiply the quantised values in
    # bf16 (the FP4 weight-stream kernels), so the bf16 peak applies
    w4a8_mx = w4a8 and T >= TILED_MIN_TOKENS
    w4a8_stream = w4a8 and 1 < T < TILED_MIN_TOKENS
    peak = FP8_PEAK_TFLOPS if w4a8_mx else BF16_PEAK_TFLOPS
    desc = moe.MoeLayerDesc.make(H, I, E, k, ns)

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    layers, host = [], []
    for li in range(L):
        x_bits, wr_bits, bias = synth.make_router_inputs(name, seed=args.seed, layer=li)
        layers.append(moe.MoELayer(desc, dev_bf16(wr_bits), torch.from_numpy(bias).cuda(), experts[li],
                                   w4a8=w4a8))
        host.append((x_bits, wr_bits, bias))
    # the activations: shared by the layers where the workload's recipe
    # shares them (i.i.d. and Zipf routing), one per layer where it does not
    # (uniform routing fits x to each layer's router)
    x_of = []
    for li in range(L):
        same = li > 0 and np.array_equal(host[li][0], host[0][0])
        x_of.append(x_of[0] if same else dev_bf16(host[li][0]))
    buf = moe.Buffers(desc, T, fp8=w4a8)
    torch.cuda.synchronize()

    def step(i):
        layers[i % L].forward(x_of[i % L], buf)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()

    # ---- whole steps in a HIP graph --------------------------------------
    cap = torch.cuda.Stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if args.eager:
        torch.cuda.synchronize()
        e0.record()
        for i in range(K):
            step(i)
        e1.record()
        torch.cuda.synchronize()
    else:
        graph = torch.cuda.CUDAGraph()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                for i in range(K):
                    step(i)
        torch.cuda.current_stream().wait_stream(cap)
        graph.replay()
        torch.cuda.synchronize()
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        del graph
    buf.check_decode()  # raises if a wait of the one-launch decode step timed out
    ms_per_step = e0.elapsed_time(e1) / K

    # ---- dominant kernel: back-to-back launches, HIP events ----------------
    # Route and permute every resident layer once into its own index buffers,
    # then capture nk gate/up launches (layer i mod L) in a graph and time one
    # replay with events on the launch stream.  At one token the step is one
    # launch: the kernel timed is the whole layer.
    one_launch = T == 1 and layers[0].one_launch(1)
    if T == 1 and not one_launch:
        raise SystemExit("the one-launch decode step is not supported on this device")
    nk = args.kernel_launches or (8 * L if T >= 1024 else max(200, 8 * L))
    per_layer = []
    for li in range(L):
        lay = layers[li]
        b = moe.Buffers(desc, T, fp8=w4a8)
        if w4a8_stream:  # the layer's quantised activations, as forward makes them
            moe.moe_act_quant_fp8_dequant(T, H, x_of[li], b.xq, b.xqs, b.xdq)
        elif w4a8:
            moe.moe_act_quant_fp8(T, H, x_of[li], b.xq, b.xqs)
        moe.moe_route(desc, T, x_of[li], lay.w_router, lay.gate_bias, b.logits, b.topk_idx, b.topk_w)
        moe.moe_permute(desc, T, b.topk_idx, b.group_offsets, b.sorted_token, b.row_of_slot, ws=b.ws)
        per_layer.append((b.group_offsets, b.sorted_token, b))
    torch.cuda.synchronize()
    bytes_, flops, lbytes, lflops, touched_all = [], [], [], [], []
    for li in range(L):
        counts = np.diff(per_layer[li][0].cpu().numpy())
        touched = int((counts > 0).sum())
        touched_all.append(touched)
        R = int(counts.sum())
        lb, lf = layer_work(T, H, E, I, counts, fmt)
        lbytes.append(lb)
        lflops.append(lf)
        # algorithmic bytes of the timed kernel: codes + scales of every
        # touched group, the T activation rows read once, the R SwiGLU rows
        # written; at one token the whole layer (router rows, gate/up and
        # down codes + scales, x read, h and out written)
        if one_launch:
            bytes_.append(E * H * 2 + touched * (3 * I * H // 2 + 2 * I * scale_bytes_per_row(H, fmt)
                                                 + H * scale_bytes_per_row(I, fmt)) + H * 2
                          + R * I * 2 + H * 2)
            flops.append(2.0 * E * H + 2.0 * R * 3 * I * H)
        else:
            act_bytes = T * H + T * H // 128 if w4a8_mx else T * H * 2  # fp8 codes + scales, or bf16
            bytes_.append(touched * (2 * I * H // 2 + 2 * I * scale_bytes_per_row(H, fmt)) + act_bytes
                          + R * I * 2)
            flops.append(2.0 * R * 2 * I * H)
    kb = [bytes_[i % L] for i in range(nk)]
    kf = [flops[i % L] for i in range(nk)]

    sums_of = [None] * L
    if T >= moe.MOE_TILED_MIN_TOKENS and fmt == "int4":  # the layer's row sums of x, as forward passes them
        for li in range(L):
            if li > 0 and x_of[li] is x_of[0]:
                sums_of[li] = sums_of[0]
                continue
            sums_of[li] = torch.empty((T, H // 128), dtype=torch.float32, device="cuda")
            moe.moe_row_sums(T, H, x_of[li], sums_of[li])

    def gemm13(i):
        lay, x = layers[i % L], x_of[i % L]
        if one_launch:
            lay.forward(x, buf)
            return
        offs, srt, b = per_layer[i % L]
        if w4a8_stream:
            moe.moe_mxfp4_grouped_gemm(desc, T, b.xdq, srt, T, 2 * I, H, lay.experts.w13, lay.experts.s13,
                                       offs, moe.MOE_ACT_SWIGLU, buf.h)
            return
        if w4a8:
            moe.moe_w4a8_grouped_gemm(desc, T, b.xq, b.xqs, srt, T, 2 * I, H, lay.experts.w13, lay.experts.s13,
                                      offs, moe.MOE_ACT_SWIGLU, buf.h)
            return
        if fmt == "fp4":
            moe.moe_mxfp4_grouped_gemm(desc, T, x, srt, T, 2 * I, H, lay.experts.w13, lay.experts.s13,
                                       offs, moe.MOE_ACT_SWIGLU, buf.h)
            return
        moe.moe_w4a16_grouped_gemm(desc, T, x, srt, T, sums_of[i % L], 2 * I, H, lay.experts.w13,
                                   lay.experts.s13, offs, moe.MOE_ACT_SWIGLU, buf.h)

    for i in range(L):
        gemm13(i)
    stream = torch.cuda.current_stream()
    a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if args.eager:
        torch.cuda.synchronize()
        a_ev.record(stream)
        for i in range(nk):
            gemm13(i)
        b_ev.record(stream)
        b_ev.synchronize()
    else:
        kgraph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(kgraph, stream=cap):
                for i in range(nk):
                    gemm13(i)
        torch.cuda.current_stream().wait_stream(cap)
        kgraph.replay()
        torch.cuda.synchronize()
        a_ev.record(stream)
        kgraph.replay()
        b_ev.record(stream)
        b_ev.synchronize()
        del kgraph
    buf.check_decode()
    avg = a_ev.elapsed_time(b_ev) * 1e-3 / nk
    roof = roofline(float(np.mean(kb)), float(np.mean(kf)), avg, peak)
    kname, _, kfiles = dominant_kernel(T, fmt)
    roof.update(traffic=load_traffic(kname, traffic_tag(name, fmt, kname), kfiles),
                kernel="%s (%s)" % (kname, "whole layer, one launch" if one_launch else "gate/up, SwiGLU"),
                avg_launch_us=round(avg * 1e6, 2), launches=nk, algorithmic_bytes=int(np.mean(kb)),
                algorithmic_flop=float(np.mean(kf)))
    layer_roof = roofline(float(np.mean(lbytes)), float(np.mean(lflops)), ms_per_step * 1e-3, peak)
    layer_roof.update(algorithmic_bytes=int(np.mean(lbytes)), algorithmic_flop=float(np.mean(lflops)))
    rec = {"value": round(T / (ms_per_step * 1e-3), 1), "unit": "tokens/s", "steps": K,
           "dtype": "fp8" if w4a8_mx else "bf16",
           "ms_per_step": round(ms_per_step, 5),
           "config": {"workload": name, "tokens": T, "hidden": H, "routed_experts": E, "top_k": k,
                      "shared_experts": ns, "inter": I, "group_size": 128 if fmt == "int4" else 32,
                      "weights": "int4 g128 fp16 scales" if fmt == "int4" else "fp4 e2m1, ue8m0 scale per 32",
                      "activations": "fp8 e4m3, ue8m0 scale per token per 128" if w4a8 else "bf16",
                      "resident_layers": L, "graph": not args.eager,
                      "experts_touched_per_layer": round(float(np.mean(touched_all)), 1)},
           "roofline": roof, "layer_roofline": layer_roof}
    del layers, buf, per_layer, x_of, sums_of
    return rec, host


def main():
    args = parse()
    if args.ingest_pmc:
        ingest_pmc(args.workload, *args.ingest_pmc, fmt=args.format)
        return
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU; --gpus %d is not supported by this build "
              "(the multi-GPU layout is design only)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import w4a16_routed_expert_moe_amd as moe

    torch.cuda.set_device(0)
    head = args.workload
    if head == FP8_PROJ:  # the projection alone, for counter runs
        rec = run_fp8_proj(args)
        print("# fp8_block: %.5f ms/step, %.1f tokens/s, %s %.1f%% (%s)" %
              (rec["ms_per_step"], rec["value"], rec["roofline"]["bound"], 100 * rec["roofline"]["frac"],
               rec["roofline"]["kernel"]), file=sys.stderr, flush=True)
        if args.calib_copy_mib:
            calib_copy(args.calib_copy_mib)
        print(json.dumps(rec), flush=True)
        return
    names = [head] if args.only else [head] + [w for w in ALL_WORKLOADS if w != head]
    n_layers = {w: (args.layers if (w == head and args.layers) else DEFAULT_LAYERS[w]) for w in names}
    wl = synth.WORKLOADS[head]
    H, E, I, ns = wl["H"], wl["E"], wl["I"], wl["n_shared"]
    G = E + ns

    # ---- resident expert weights ------------------------------------------
    # Layer li's experts are the same for every workload (the seeded
    # generator keys them by layer), so the workloads share one resident set
    # of max(layers) layers (43 at the stack: 144.9 GB of HBM); each workload
    # brings its own router, bias and activations.
    def resident(fmt):
        scratch = torch.empty(G * 2 * I * H // 2, dtype=torch.uint8, device="cuda")
        ex = [moe.generate_weights(args.seed, li, G, H, I, scratch=scratch, fmt="int4" if fmt == "int4" else "fp4")
              for li in range(max(n_layers.values()))]
        del scratch
        torch.cuda.synchronize()
        return ex

    def report(key, rec):
        print("# %s: %.5f ms/step, %.1f tokens/s, %s %.1f%% (%s)" %
              (key, rec["ms_per_step"], rec["value"], rec["roofline"]["bound"],
               100 * rec["roofline"]["frac"], rec["roofline"]["kernel"]), file=sys.stderr, flush=True)

    experts = resident(args.format)
    results, host0 = {}, None
    for w in names:
        steps = args.steps if (w == head and args.steps) else DEFAULT_STEPS[w]
        rec, host = run_workload(w, args, experts, steps, args.warmup, n_layers[w], args.format)
        results[w] = rec
        if w == head:
            host0 = host
        report(w, rec)
        torch.cuda.synchronize()
    extra = {}
    if not args.only:
        # the same workloads with fp8 activations (W4A8: the release's FP4
        # experts, e4m3 activations per token per 128), then the FP8_BLOCK
        # projection GEMM
        if args.format != "w4a8":
            del experts
            torch.cuda.empty_cache()
            experts = resident("w4a8")
            for w in names:
                rec, _ = run_workload(w, args, experts, DEFAULT_STEPS[w], args.warmup, n_layers[w], "w4a8")
                extra["w4a8/" + w] = rec
                report("w4a8/" + w, rec)
        del experts
        torch.cuda.empty_cache()
        rec = run_fp8_proj(args)
        extra["fp8_block/" + rec["config"]["workload"]] = rec
        report("fp8_block", rec)

    if args.calib_copy_mib:
        calib_copy(args.calib_copy_mib)

    # ---- CPU oracle on a bounded sample -----------------------------------
    cpu = None
    if args.cpu_seconds > 0:
        w = synth.WORKLOADS[head]
        cpu = cpu_baseline(head, args.seed, host0, n_layers[head], w["T"], H, E, w["k"], I, ns,
                           args.cpu_seconds, args.format)

    hr = results[head]
    rec = {
        "metric": METRIC, "value": hr["value"], "unit": "tokens/s", "n_gpus": 1, "steps": hr["steps"],
        "warmup": args.warmup, "ms_per_step": hr["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": hr["dtype"], "data": "synthetic",
        "config": hr["config"],
        "roofline": hr["roofline"],
        "layer_roofline": hr["layer_roofline"],
        "cpu_baseline": cpu,
        "configs": dict({w: results[w] for w in names if w != head}, **extra),
    }
    print(json.dumps(rec), flush=True)


def calib_copy(mib):
    """One plain device copy of ``mib`` MiB: the counter calibration that
    ingest_pmc scales FETCH_SIZE and WRITE_SIZE by."""
    import torch
    src = torch.ones(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def run_fp8_proj(args, M=8192, N=4096, K=4096):
    """The FP8_BLOCK projection GEMM at an 8192-token prefill (4096 x 4096
    weights, e4m3 with a UE8M0 scale per 128x128 block; the pages give the
    format but not the projections' shapes): a step is the activation
    quantisation plus the GEMM."""
    import torch

    import synth
    import w4a16_routed_expert_moe_amd as moe

    wc, ws = synth.fp8_block_weights(args.seed, 0, N, K)
    packed = torch.empty(N * K, dtype=torch.uint8, device="cuda")
    moe.moe_fp8_prepack(N, K, torch.from_numpy(wc.reshape(-1).copy()).cuda(), packed)
    wsd = torch.from_numpy(ws.copy()).cuda()
    x = torch.from_numpy(synth.make_x(M, K, args.seed).view(np.int16)).view(torch.bfloat16).cuda()
    xq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((M, K // 128), dtype=torch.uint8, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def quant():
        moe.moe_act_quant_fp8(M, K, x, xq, xs)

    def gemm():
        moe.moe_fp8_block_gemm(M, N, K, xq, xs, packed, wsd, out)

    def timed(fn, n):
        for _ in range(3):
            fn()
        cap = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for _ in range(n):
                    fn()
        torch.cuda.current_stream().wait_stream(cap)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) * 1e-3 / n

    def eager(fn, n):  # counter runs: plain launches, no graph
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) * 1e-3 / n

    n = 40
    run = eager if args.eager else timed
    step_s = run(lambda: (quant(), gemm()), n)
    gemm_s = run(gemm, n)
    flop = 2.0 * M * N * K
    gbytes = N * K + (N // 128) * (K // 128) + M * K + M * (K // 128) + M * N * 2
    roof = roofline(gbytes, flop, gemm_s, FP8_PEAK_TFLOPS)
    _, _, files = dominant_kernel(0, "fp8_block")
    roof.update(traffic=load_traffic("k_mx_gemm", FP8_PROJ, files), kernel="k_mx_gemm<0,0> (fp8 x fp8, block scales)",
                avg_launch_us=round(gemm_s * 1e6, 2), launches=n, algorithmic_bytes=int(gbytes),
                algorithmic_flop=flop)
    return {"value": round(M / step_s, 1), "unit": "tokens/s", "steps": n, "dtype": "fp8",
            "ms_per_step": round(step_s * 1e3, 5),
            "config": {"workload": FP8_PROJ, "tokens": M, "N": N, "K": K,
                       "weights": "fp8 e4m3, ue8m0 scale per 128x128 block",
                       "activations": "fp8 e4m3, ue8m0 scale per token per 128 (quantised in the step)"},
            "roofline": roof}


def cpu_cores():
    """Host threads this process may use (the machine's CPU share: at most 16)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(workload, seed, host, L, T, H, E, k, I, ns, budget_s, fmt="int4"):
    """The oracle as it stands on a bounded sample of the workload, on every
    host core this process may use: independent whole-layer forwards of the
    first min(T, 4) tokens of a layer (routing, expert MLPs of the chosen
    groups with on-the-fly dequantisation, combine), one per worker thread
    at a time (the oracle's own threads set to 1 in each worker; ctypes
    releases the interpreter lock).  Weight generation is not timed.
    Returns tokens/s of the oracle."""
    import concurrent.futures as cf

    import oracle
    import synth

    cores = cpu_cores()
    per_tok = max(1, min(T, 4))
    n_lay = min(L, 2)
    gen = synth.expert_weights if fmt == "int4" else synth.fp4_expert_weights
    weights = {}
    for li in range(n_lay):  # untimed: the groups each sample's routing needs
        x_bits, wr_bits, bias = host[li]
        idx, _ = oracle.select(oracle.router_logits(x_bits[:per_tok], wr_bits), bias, k)
        for g in sorted(set(int(g) for g in idx.ravel()) | ({E} if ns else set())):
            weights[(li, g)] = gen(seed, li, g, H, I)

    def sample(i):
        oracle.set_threads(1)
        li = i % n_lay
        x_bits, wr_bits, bias = host[li]
        toks = x_bits[:per_tok]
        logits = oracle.router_logits(toks, wr_bits)
        idx, w = oracle.select(logits, bias, k)
        oracle.token_outputs(range(per_tok), toks, idx, w, lambda g: weights[(li, g)], E, ns, fmt=fmt)
        return per_tok

    t0 = time.perf_counter()
    sample(0)  # one sample alone sizes the run
    t1 = time.perf_counter() - t0
    n = cores * max(1, int(round(budget_s / max(t1, 1e-3))))
    with cf.ThreadPoolExecutor(max_workers=cores) as ex:
        t0 = time.perf_counter()
        done = sum(ex.map(sample, range(n)))
        wall = time.perf_counter() - t0
    oracle.set_threads(cores)
    return {"value": round(done / wall, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "%d whole-layer forwards of %d token(s) of the %s workload (%d layers of its "
                      "rotation), %d at a time on %d host threads, %.1f s wall; one forward alone "
                      "took %.2f s" % (n, per_tok, workload, n_lay, cores, cores, wall, t1)}


if __name__ == "__main__":
    main()
