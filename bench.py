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

Prints one JSON line.  ``--gpus N`` with N > 1 is refused: this build runs on
one GPU.
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

DEFAULT_LAYERS = {"decode1": 8, "decode64": 4, "prefill8k": 2, "stack43": 43}
DEFAULT_STEPS = {"decode1": 200, "decode64": 100, "prefill8k": 20, "stack43": 86}
TILED_MIN_TOKENS = 384  # the grouped GEMM takes its LDS-tiled kernel from here on
CSRC = os.path.join(ROOT, "w4a16_routed_expert_moe_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def dominant_kernel(T, fmt="int4"):
    """(name, rocprofv3 name prefix, source files) of the kernel priced against
    its roofline at T tokens: the one-launch decode step at one token (the
    whole layer), else the gate/up GEMM."""
    common = ["moe_common.h", "moe_gemm_common.h"]
    if fmt == "fp4":
        if T == 1:
            return ("k_mxfp4_decode_token", "k_mxfp4_decode_token<",
                    common + ["moe_route_common.h", "moe_decode.hip"])
        if T >= TILED_MIN_TOKENS:
            return "k_mxfp4_tiled", "k_mxfp4_tiled<1,", common + ["moe_gemm_tiled.hip"]
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
                       "python3 bench.py --workload %s --eager --calib-copy-mib 256 --cpu-seconds 0" % workload,
                       "rocprofv3 --pmc WRITE_SIZE (same)",
                       "python3 bench.py --workload %s --ingest-pmc <fetch csv> <write csv>" % workload]}
    if fmt != "int4":
        rec["command"] = [c.replace("--workload", "--format %s --workload" % fmt) for c in rec["command"]]
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_file(kernel, workload), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode1", choices=list(DEFAULT_LAYERS))
    ap.add_argument("--layers", type=int, default=None, help="resident layers in the rotation")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--kernel-launches", type=int, default=None,
                    help="launches of the dominant kernel timed with events")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step directly instead of through HIP graphs (for counter runs)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic summary of the dominant kernel from two counter runs")
    ap.add_argument("--format", default="int4", choices=["int4", "fp4"],
                    help="expert weights: INT4 with fp16 scales per 128 (the layer's format), or the "
                         "release's FP4 (E2M1, UE8M0 scale per 32)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample (0 = skip)")
    return ap.parse_args()


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
    wl = synth.WORKLOADS[args.workload]
    T, H, E, k, I, ns = wl["T"], wl["H"], wl["E"], wl["k"], wl["I"], wl["n_shared"]
    G = E + ns
    L = args.layers or DEFAULT_LAYERS[args.workload]
    K = args.steps or DEFAULT_STEPS[args.workload]
    W = args.warmup
    desc = moe.MoeLayerDesc.make(H, I, E, k, ns)

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    # ---- resident layers ------------------------------------------------
    layers, host = [], []
    scratch = torch.empty(G * 2 * I * H // 2, dtype=torch.uint8, device="cuda")
    for li in range(L):
        x_bits, wr_bits, bias = synth.make_router_inputs(args.workload, seed=args.seed, layer=li)
        experts = moe.generate_weights(args.seed, li, G, H, I, scratch=scratch, fmt=args.format)
        layers.append(moe.MoELayer(desc, dev_bf16(wr_bits), torch.from_numpy(bias).cuda(), experts))
        host.append((x_bits, wr_bits, bias))
    del scratch
    x = dev_bf16(host[0][0])  # every layer reads the same activations
    buf = moe.Buffers(desc, T)
    torch.cuda.synchronize()

    def step(i):
        layers[i % L].forward(x, buf)

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
    ms_per_step = e0.elapsed_time(e1) / K
    value = T / (ms_per_step * 1e-3)

    # ---- dominant kernel: back-to-back launches, HIP events ----------------
    # Route and permute every resident layer once into its own index buffers,
    # then capture nk gate/up launches (layer i mod L) in a graph and time one
    # replay with events on the launch stream.  At one token the step is one
    # launch: the kernel timed is the whole layer.
    fmt = args.format
    one_launch = T == 1 and layers[0].one_launch(1)
    if T == 1 and not one_launch:
        raise SystemExit("the one-launch decode step is not supported on this device")
    nk = args.kernel_launches or (8 * L if T >= 1024 else max(200, 8 * L))
    per_layer = []
    for li in range(L):
        lay = layers[li]
        b = moe.Buffers(desc, T)
        moe.moe_route(desc, T, x, lay.w_router, lay.gate_bias, b.logits, b.topk_idx, b.topk_w)
        moe.moe_permute(desc, T, b.topk_idx, b.group_offsets, b.sorted_token, b.row_of_slot)
        per_layer.append((b.group_offsets, b.sorted_token))
    torch.cuda.synchronize()
    bytes_, flops = [], []
    for li in range(L):
        counts = np.diff(per_layer[li][0].cpu().numpy())
        touched = int((counts > 0).sum())
        R = int(counts.sum())
        # algorithmic bytes: codes + scales of every touched group, the T
        # activation rows read once, the R SwiGLU rows written
        if one_launch:
            # the whole layer: router rows, gate/up and down codes + scales of
            # the touched groups, x read, h and out written
            bytes_.append(E * H * 2 + touched * (3 * I * H // 2 + 2 * I * scale_bytes_per_row(H, fmt)
                                                 + H * scale_bytes_per_row(I, fmt)) + H * 2
                          + R * I * 2 + H * 2)
            flops.append(2.0 * E * H + 2.0 * R * 3 * I * H)
        else:
            bytes_.append(touched * (2 * I * H // 2 + 2 * I * scale_bytes_per_row(H, fmt)) + T * H * 2
                          + R * I * 2)
            flops.append(2.0 * R * 2 * I * H)
    bytes_ = [bytes_[i % L] for i in range(nk)]
    flops = [flops[i % L] for i in range(nk)]

    xs = None
    if T >= moe.MOE_TILED_MIN_TOKENS and fmt == "int4":  # the layer's row sums of x, as forward passes them
        xs = torch.empty((T, H // 128), dtype=torch.float32, device="cuda")
        moe.moe_row_sums(T, H, x, xs)

    def gemm13(i):
        lay = layers[i % L]
        if one_launch:
            lay.forward(x, buf)
            return
        offs, srt = per_layer[i % L]
        if fmt == "fp4":
            moe.moe_mxfp4_grouped_gemm(desc, T, x, srt, T, 2 * I, H, lay.experts.w13, lay.experts.s13,
                                       offs, moe.MOE_ACT_SWIGLU, buf.h)
            return
        moe.moe_w4a16_grouped_gemm(desc, T, x, srt, T, xs, 2 * I, H, lay.experts.w13, lay.experts.s13,
                                   offs, moe.MOE_ACT_SWIGLU, buf.h)

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
    if args.calib_copy_mib:
        src = torch.ones(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    durs = [a_ev.elapsed_time(b_ev) * 1e-3 / nk]
    avg = float(np.mean(durs))
    gbs = float(np.mean(bytes_)) / avg / 1e9
    tfs = float(np.mean(flops)) / avg / 1e12
    intensity = float(np.mean(flops)) / float(np.mean(bytes_))
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if intensity < ridge:
        roof = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(gbs / HBM_PEAK_GBS, 4))
    else:
        roof = dict(bound="mfma", achieved=round(tfs, 1), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(tfs / BF16_PEAK_TFLOPS, 4))
    kname, _, kfiles = dominant_kernel(T, fmt)
    roof.update(traffic=load_traffic(kname, args.workload, kfiles),
                kernel="%s (%s)" % (kname, "whole layer, one launch" if one_launch else "gate/up, SwiGLU"),
                avg_launch_us=round(avg * 1e6, 2),
                launches=nk, algorithmic_bytes=int(np.mean(bytes_)),
                algorithmic_flop=float(np.mean(flops)))

    # ---- CPU oracle on a bounded sample -----------------------------------
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(args.workload, args.seed, host, L, T, H, E, k, I, ns, args.cpu_seconds, fmt)

    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "hidden": H, "routed_experts": E,
                   "top_k": k, "shared_experts": ns, "inter": I, "group_size": 128 if fmt == "int4" else 32,
                   "weights": "int4 g128 fp16 scales" if fmt == "int4" else "fp4 e2m1, ue8m0 scale per 32",
                   "resident_layers": L, "graph": not args.eager},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def cpu_baseline(workload, seed, host, L, T, H, E, k, I, ns, budget_s, fmt="int4"):
    """The oracle as it stands on a bounded sample: whole-layer forwards of
    single tokens (decode) or of a slice of the batch, timed without input
    generation.  Returns tokens/s of the oracle."""
    import oracle
    import synth

    oracle.set_threads(1)
    per_tok = max(1, min(T, 4))
    done_tokens, spent, li = 0, 0.0, 0
    while spent < budget_s and li < 64:
        x_bits, wr_bits, bias = host[li % L]
        toks = x_bits[:per_tok]
        t0 = time.perf_counter()
        logits = oracle.router_logits(toks, wr_bits)
        idx, w = oracle.select(logits, bias, k)
        t_route = time.perf_counter() - t0
        groups = sorted(set(int(g) for g in idx.ravel()) | ({E} if ns else set()))
        gen = synth.expert_weights if fmt == "int4" else synth.fp4_expert_weights
        weights = {g: gen(seed, li % L, g, H, I) for g in groups}
        t0 = time.perf_counter()
        oracle.token_outputs(range(per_tok), toks, idx, w, lambda g: weights[g], E, ns, fmt=fmt)
        spent += t_route + time.perf_counter() - t0
        done_tokens += per_tok
        li += 1
    return {"value": round(done_tokens / spent, 3), "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": "%d whole-layer token forwards (%d per layer, %d layers of the %s rotation), "
                      "%.1f s of oracle time, one thread" %
                      (done_tokens, per_tok, li, workload, spent)}


if __name__ == "__main__":
    main()
