#!/usr/bin/env python3
"""Benchmark of the MXFP4 MoE expert layer on one MI355X.

Metric: MoE expert-layer tokens/s on the 256-token verify step (32 sequences
x a DFlash block of 8 tokens; d_model 4096, d_ff 1536, 64 experts, top-8,
router logits with a per-expert N(0, 0.5) bias), with the achieved HBM
GB/s of the layer and of its dominant kernel against the 8 TB/s peak.

One step = one forward call of the whole path (routing, permutation, gate/up
+ SwiGLU, down, combine) over the synthetic batch; inputs and packed weights
are resident in HBM before the timed region.  Consecutive steps rotate over
several copies of the weights so that no step finds another step's weights
in the 256 MB last-level cache.  The CPU oracle is timed on a bounded token
sample as a reported baseline (rank 0, one GPU only).

Beside the metric, the line carries: per-stage times (HIP events), p10 /
p50 / p90 of single calls, the GPU's measured streaming-read and MFMA
rates (library probes) with the roofline fraction against them, and for
the verify workloads the DFlash acceptance pass over the batch's sequences
as its own figure (with the oracle's time on the same batch).  --graph adds
the same calls replayed from captured HIP graphs.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MXFP4_PEAK_TFLOPS = 10100.0    # MI355X dense FP4/FP6 matrix peak
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 matrix peak (the rate of FP8 x FP4 scaled MFMA)
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
WNAMES = ("w_gate", "w_gate_scale", "w_up", "w_up_scale", "w_down", "w_down_scale")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def weight_shapes(w):
    return {"w_gate": (w.E, w.f, w.d // 2), "w_gate_scale": (w.E, w.f, w.d // 32),
            "w_up": (w.E, w.f, w.d // 2), "w_up_scale": (w.E, w.f, w.d // 32),
            "w_down": (w.E, w.d, w.f // 2), "w_down_scale": (w.E, w.d, w.f // 32)}


def pack_on_gpu(w, copies, moe, torch):
    """Generate fp32 expert weights (synth), pack them with the library's
    quantiser on the GPU, convert to the tiled layout the forward path reads,
    and clone into `copies` independent copies."""
    import synth
    shapes = weight_shapes(w)
    packed = {n: torch.empty(s, dtype=torch.uint8, device="cuda") for n, s in shapes.items()}
    for e, g, u, dn in synth.all_expert_weights_f32(w):
        for name, m in (("w_gate", g), ("w_up", u), ("w_down", dn)):
            t = torch.from_numpy(m).cuda()
            moe.quantize_weights(t, packed=packed[name][e], scales=packed[name + "_scale"][e])
    tiled = moe.tile_expert_weights(packed)
    del packed
    torch.cuda.synchronize()
    out = [tiled]
    for _ in range(copies - 1):
        out.append({n: t.clone() for n, t in tiled.items()})
    torch.cuda.synchronize()
    return out


def cpu_baseline(w, acts, ntok, router_bits=None, threads=None):
    """The oracle, as it stands, on the first `ntok` tokens (oracle-packed weights);
    with `router_bits` (bf16 [E, d]) the logits come from the oracle's router
    projection, timed with the layer.  threads: OpenMP threads of the oracle
    (default: up to 16, the host share of one GPU)."""
    import numpy as np
    import oracle
    import synth
    from concurrent.futures import ThreadPoolExecutor
    pack_threads = min(16, os.cpu_count() or 1)
    threads = pack_threads if threads is None else threads
    x, lg = acts["x_bf16"][:ntok], acts["logits"][:ntok]
    t_router = 0.0
    if router_bits is not None:
        t0 = time.perf_counter()
        lg = oracle.router_logits(x, router_bits)[0].astype(np.float32)
        t_router = time.perf_counter() - t0
    ids, _ = oracle.route(lg, w.k)
    need = [int(e) for e in np.unique(ids)]
    wts = {n: np.zeros(s, np.uint8) for n, s in weight_shapes(w).items()}

    def job(e):
        g, u, dn = synth.expert_weights_f32(w, e)
        for name, m in (("w_gate", g), ("w_up", u), ("w_down", dn)):
            p, s = oracle.quant_mxfp4(m)
            wts[name][e] = p
            wts[name + "_scale"][e] = s

    with ThreadPoolExecutor(pack_threads) as ex:
        list(ex.map(job, need))
    t0 = time.perf_counter()
    r = oracle.moe_forward(x, lg, wts, w.k, nthreads=threads)
    dt = time.perf_counter() - t0 + t_router
    return {"value": ntok / dt, "unit": "tokens/s", "cores": int(r["threads"]), "kind": "oracle",
            "sample": f"first {ntok} of {w.T} tokens of {w.name}, all {w.k} experts each"
                      f"{', router projection included' if router_bits is not None else ''}; "
                      f"fp64 C oracle, {'OpenMP over tokens' if threads > 1 else 'one thread'}; "
                      f"{dt:.2f} s wall; {cpu_model()}, {os.cpu_count()} logical CPUs visible"}


def time_graph_replay(layers, x, lg, out, ws, wr, args, torch):
    """The timed loop again, each call replayed from a HIP graph captured
    once per weight copy (same buffers, so the replays do the same work)."""
    side = torch.cuda.Stream()                      # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for L in layers:
            L(x, lg, out=out, workspace=ws, w_router=wr)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for L in layers:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            L(x, lg, out=out, workspace=ws, w_router=wr)
        graphs.append(g)
    for i in range(args.warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    log(f"graph replay: {ms:.4f} ms per call")
    return {"ms_per_step": ms, "graphs": len(graphs)}


def measure_peaks(moe, torch):
    """What this GPU sustains: a 4 GiB streaming read and the MFMA issue
    rates of the three instructions the path uses (the library's probes),
    each timed over 5 launches with HIP events on the launch stream."""
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    src = torch.ones(4 << 30, dtype=torch.uint8, device="cuda")

    def rate(kind, reps, src=None):
        moe.probe(kind, src=src, reps=reps, sink=sink)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            work = moe.probe(kind, src=src, reps=reps, sink=sink)
        e1.record()
        torch.cuda.synchronize()
        return work / (e0.elapsed_time(e1) / 5 * 1e-3)

    out = {"stream_read_GBps": rate(moe.PROBE_STREAM, 0, src) / 1e9}
    del src
    # constant operands, then random operands that change every MFMA (the
    # clock the chip holds under its power limit depends on the data)
    for kind, name, reps, nominal in (
            (moe.PROBE_MFMA_BF16, "mfma_bf16_16x16x32", 250, BF16_PEAK_TFLOPS),
            (moe.PROBE_MFMA_FP8_FP4, "mfma_fp8xfp4_16x16x128", 125, FP8_PEAK_TFLOPS),
            (moe.PROBE_MFMA_FP4_FP4, "mfma_fp4xfp4_16x16x128", 250, MXFP4_PEAK_TFLOPS),
            (moe.PROBE_MFMA_BF16_RANDOM, "mfma_bf16_16x16x32_random", 250, BF16_PEAK_TFLOPS),
            (moe.PROBE_MFMA_FP8_FP4_RANDOM, "mfma_fp8xfp4_16x16x128_random", 125, FP8_PEAK_TFLOPS),
            (moe.PROBE_MFMA_FP4_FP4_RANDOM, "mfma_fp4xfp4_16x16x128_random", 250, MXFP4_PEAK_TFLOPS)):
        tf = rate(kind, reps) / 1e12
        out[name] = {"TFLOPs": tf, "nominal_TFLOPs": nominal, "frac_of_nominal": tf / nominal}
    log("measured peaks: " + ", ".join(f"{k} {v if isinstance(v, float) else v['TFLOPs']:.0f}" for k, v in out.items()))
    return out


def per_call_percentiles(call, steps, torch):
    """p10 / p50 / p90 of single calls, each between its own HIP events."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(ev):
        a.record()
        call(i)
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    pick = lambda q: ms[min(len(ms) - 1, int(q * len(ms)))]
    return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline_accept(inp):
    """The oracle's acceptance pass over the same batch (one thread)."""
    import oracle
    args = [inp[k] for k in ("draft", "p_draft", "p_target", "u", "r")]
    reps, t0 = 0, time.perf_counter()
    while reps < 3 or time.perf_counter() - t0 < 1.0:
        oracle.dflash_accept(*args)
        reps += 1
    dt = (time.perf_counter() - t0) / reps
    B = inp["draft"].shape[0]
    return {"value": B / dt, "unit": "sequences/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole batch ({B} sequences), {reps} calls; {dt * 1e3:.2f} ms per call"}


def kernel_path(moe, w, mx8):
    """The kernels a forward call of this workload runs: the dense FP8 x FP4
    kernels in MXFP8 mode; for bf16 activations the fused path (the library's
    default; MOE_MXFP4_PATH=stream selects the per-phase launches), in its
    ticketed form where the batch has more pairs than experts, else its
    persistent form, up to FUSED_MAX_PAIRS pairs."""
    if mx8:
        return "dense"
    path = os.environ.get("MOE_MXFP4_PATH") or "fused"
    if path == "stream" or w.P > moe.FUSED_MAX_PAIRS:
        return "stream"
    # one verify block (at most 64 pairs over at most 128 experts, no more
    # pairs than experts, at most 1024 logits): routing, permutation and both
    # projections in one launch, then the combine
    if path == "fused" and w.E <= 128 and w.P <= 64 and w.P <= w.E and w.T * w.E <= 1024:
        return "fused (routing in the expert launch)"
    return "fused (ticketed)" if w.P > w.E else "fused (persistent)"


def measured_traffic(workload, mx8, root=None, path=None):
    """Bytes beyond L2 per launch of the dominant kernel (FETCH_SIZE +
    WRITE_SIZE, each scaled by what it reads for a plain copy of known size;
    includes hits in the last-level cache, so it bounds HBM bytes from
    above) from the committed counter summary of this workload, or None when
    there is none or the kernel's source file changed since the counters were
    taken.  root: the repository (default: here); path "stream": the
    per-phase path's summary (the default path's otherwise)."""
    import hashlib
    root = root or os.path.dirname(os.path.abspath(__file__))
    # the per-phase path's counters sit in a summary of their own
    suffix = "_stream" if path == "stream" else ""
    summary = os.path.join(root, "profiles", f"beyond_l2_bytes_{workload}{suffix}.md")
    if not os.path.exists(summary):
        return None
    fields = {}
    for line in open(summary):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    # the kernel's source files (comma-separated: the kernel file and the
    # headers it is built from), hashed as one concatenation in that order
    srcs = [os.path.join(root, f.strip().strip("`")) for f in fields.get("kernel source", "?").split(",")]
    if not all(os.path.exists(f) for f in srcs) or "traffic bytes per launch" not in fields:
        return None
    h = hashlib.sha256()
    for f in srcs:
        h.update(open(f, "rb").read())
    if fields.get("kernel source sha256") != h.hexdigest():
        return None
    return float(fields["traffic bytes per launch"])


def event_spacing_us(torch, n=64):
    """Median time between two HIP events recorded back to back on the
    current stream (after a small kernel, as between the stages of a call):
    what every per-stage event time carries on top of its kernels."""
    buf = torch.empty(1024, device="cuda")
    pairs = []
    for _ in range(n):
        buf.zero_()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        b.record()
        pairs.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in pairs)
    return 1e3 * ms[len(ms) // 2]


def time_accept(w, args, moe, torch, np, synth):
    """The acceptance pass over the batch's sequences: every row it reads is
    an HBM stream (4 bytes per vocabulary entry), so it is priced against HBM."""
    B, G, V = w.T // 8, 8, synth.DFLASH_VOCAB
    inp = synth.dflash_batch(B, G, V, seed=w.seed + 7)
    dev0 = [torch.from_numpy(inp[k]).cuda() for k in ("draft", "p_draft", "p_target", "u", "r")]
    # copies at distinct addresses, rotated so that the rows a call reads
    # (about 30 MB) are not still in the 256 MB last-level cache from the
    # previous calls: 12 copies cycle 360 MB of rows
    copies = [dev0] + [[t.clone() for t in dev0] for _ in range(args.accept_copies - 1)]
    n_acc = torch.empty(B, dtype=torch.int32, device="cuda")
    tok = torch.empty(B, dtype=torch.int32, device="cuda")
    wsa = torch.empty(moe.dflash_workspace_bytes(B, V), dtype=torch.uint8, device="cuda")

    def timed(rotate):
        for i in range(args.warmup):
            moe.dflash_accept(*copies[i % len(copies) if rotate else 0], n_accepted=n_acc, next_token=tok,
                              workspace=wsa)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            moe.dflash_accept(*copies[i % len(copies) if rotate else 0], n_accepted=n_acc, next_token=tok,
                              workspace=wsa)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.steps

    us = timed(True)
    n = n_acc.cpu().numpy()
    # rows streamed: p_target and p_draft at the rejected position, or p_target[G]
    rows = int(np.where(n < G, 2, 1).sum())
    nbytes = rows * V * 4 + B * G * (4 + 4 + 2 * 64) + B * (4 + 4 + 4 + 4)
    gbs = nbytes / (us * 1e-6) / 1e9
    log(f"dflash acceptance: {us:.1f} us per call, {gbs:.0f} GB/s, mean accepted {n.mean():.2f}")
    return {"workload": f"{B} sequences x block {G}, vocabulary {V}, float32 distributions",
            "us_per_call": us, "input_copies": len(copies), "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": nbytes, "mean_accepted": float(n.mean()),
            "whole_block_accepted": float((n == G).mean())}, inp


def parse_args(argv=None):
    """The command line (argv: a list of arguments, default sys.argv[1:])."""
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="verify_32seq")
    ap.add_argument("--tokens", type=int, default=None,
                    help="batch of this many tokens with the workload's model and routing recipe (a batch-size "
                         "sweep; the named workload's own size by default)")
    ap.add_argument("--copies", type=int, default=3, help="weight copies rotated across steps")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed forward calls for at least this long before the warmup steps (reported as "
                         "'settle'): after the host-side setup the GPU needs tens of ms of sustained work to "
                         "reach its steady clocks; 0 disables")
    ap.add_argument("--path", choices=("stream", "fused_launches", "fused"), default=None,
                    help="kernel path of the bf16 workloads (MOE_MXFP4_PATH): one launch per phase; routing, "
                         "one launch of both projections and the combine; or that with the whole layer in one "
                         "launch for a single verify block; default: the library's (fused)")
    ap.add_argument("--cpu-tokens", type=int, default=128)       # about 10 s of oracle time on 16 cores
    ap.add_argument("--cpu-tokens-1thread", type=int, default=8,
                    help="tokens of the single-threaded oracle leg (8-, 256-token verify and tiny workloads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--with-router", action="store_true",
                    help="time the forward call with the router projection in front (logits = x W_router^T "
                         "computed inside the call) instead of taking the logits as input")
    ap.add_argument("--no-accept", dest="with_accept", action="store_false",
                    help="skip timing the DFlash verify acceptance (rejection sampling) of the batch's sequences "
                         "over a full vocabulary, which is otherwise reported as its own figure")
    ap.add_argument("--with-accept", dest="with_accept", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--graph", action="store_true",
                    help="also time the same calls replayed from captured HIP graphs (one per weight copy): the "
                         "difference to the eager time is what launching costs")
    ap.add_argument("--no-peaks", dest="peaks", action="store_false",
                    help="skip measuring this GPU's streaming-read rate and MFMA issue rates (library probes), "
                         "against which the roofline fraction is otherwise reported too")
    ap.add_argument("--peaks", dest="peaks", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--accept-copies", type=int, default=12,
                    help="input copies rotated across acceptance calls")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the measurements, run a plain device copy (torch.neg, float32) of this many "
                         "MiB: the reference dispatch for scaling HBM byte counters")
    return ap.parse_args(argv)


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(no collectives, no sharding); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import mxfp4_expert_ffn_amd as moe
    import synth

    if args.path:
        os.environ["MOE_MXFP4_PATH"] = args.path
    w = synth.workload(args.workload)
    if args.tokens is not None:
        if args.tokens < 1:
            ap.error("--tokens must be positive")
        w = dataclasses.replace(w, name=f"{w.name}@{args.tokens}", T=args.tokens)
    mx8 = w.act == "mxfp8"
    torch.cuda.set_device(0)
    log(f"workload {w}")
    acts = synth.make_activations(w)
    t0 = time.time()
    wcopies = pack_on_gpu(w, args.copies, moe, torch)
    log(f"weights generated and packed on the GPU ({args.copies} copies) in {time.time() - t0:.1f} s")

    x = torch.from_numpy(acts["x_bf16"].view(np.int16)).cuda().view(torch.bfloat16)
    lg = torch.from_numpy(acts["logits"]).cuda()
    wr = None
    if args.with_router:
        wr = torch.from_numpy(synth.router_weights_bf16(w).view(np.int16)).cuda().view(torch.bfloat16)
        lg = None
    out = torch.empty((w.T, w.d), dtype=torch.bfloat16, device="cuda")
    act_mode = moe.ACT_MXFP8_E4M3 if mx8 else moe.ACT_BF16
    layers = [moe.MoeMxfp4(c, w.E, w.d, w.f, w.k, max_tokens=w.T, act_mode=act_mode) for c in wcopies]
    ws = torch.empty(layers[0].workspace_bytes(w.T), dtype=torch.uint8, device="cuda")

    # routing of this batch, from the library itself, for the byte counts
    offs = torch.empty(w.E + 1, dtype=torch.int32, device="cuda")
    layers[0](x, lg, out=out, workspace=ws, routing={"expert_offsets": offs}, w_router=wr)
    torch.cuda.synchronize()
    counts = np.diff(offs.cpu().numpy())
    touched = int((counts > 0).sum())
    per_expert = 3 * w.d * w.f * (1 / 2 + 1 / 32)
    layer_bytes = touched * per_expert + w.T * w.d * 2 + w.T * w.E * 4 + w.T * w.d * 2
    if wr is not None:
        layer_bytes += w.E * w.d * 2                  # router weights
    gateup_bytes = touched * 2 * w.f * w.d * (1 / 2 + 1 / 32) + w.T * w.d * 2
    # the fused kernel runs both projections: all expert bytes, x, and the
    # float32 per-pair outputs it writes
    fused_bytes = touched * per_expert + w.T * w.d * 2 + w.P * w.d * 4
    flops = 2.0 * w.P * 3 * w.d * w.f
    kpath = kernel_path(moe, w, mx8)

    # Settle: weight generation on the host leaves the GPU idle for seconds,
    # and the first ~100 calls after that run slower (0.160 against 0.147 ms
    # per 256-token call, one box) while the clocks ramp up.  Untimed calls
    # in batches of 8 until settle_ms have passed, then the warmup steps.
    settle_calls, ts0 = 0, time.perf_counter()
    while (time.perf_counter() - ts0) * 1e3 < args.settle_ms:
        for _ in range(8):
            layers[settle_calls % args.copies](x, lg, out=out, workspace=ws, w_router=wr)
            settle_calls += 1
        torch.cuda.synchronize()
    settle = {"calls": settle_calls, "ms": round((time.perf_counter() - ts0) * 1e3, 1),
              "why": "untimed calls before the warmup steps, until the GPU's clocks have left the idle of the "
                     "host-side setup"}

    for i in range(args.warmup):
        layers[i % args.copies](x, lg, out=out, workspace=ws, w_router=wr)
    torch.cuda.synchronize()

    # timed region: exactly `steps` forward calls
    t0 = time.perf_counter()
    for i in range(args.steps):
        layers[i % args.copies](x, lg, out=out, workspace=ws, w_router=wr)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = dt * 1e3 / args.steps

    # per-stage HIP-event timing in a second pass (events would perturb the first)
    for L in layers:
        L.stage_timing(args.steps)
    for i in range(args.steps):
        layers[i % args.copies](x, lg, out=out, workspace=ws, w_router=wr)
    torch.cuda.synchronize()
    stage_ms, ncalls = {}, 0
    for L in layers:
        t, n = L.stage_times()
        ncalls += n
        for k, v in t.items():
            stage_ms[k] = stage_ms.get(k, 0.0) + v
        L.stage_timing(0)
    stage_avg_us = {k: 1e3 * v / ncalls for k, v in stage_ms.items()}
    pct = per_call_percentiles(lambda i: layers[i % args.copies](x, lg, out=out, workspace=ws, w_router=wr),
                               args.steps, torch)
    log(f"stage averages (us): " + ", ".join(f"{k} {v:.1f}" for k, v in stage_avg_us.items()))

    # The gate/up stage's event time minus the spacing of two back-to-back
    # events (the same figure an empty stage shows) is the kernel's own
    # average duration over the calls, on the stream it is launched on.
    spacing = event_spacing_us(torch)
    gateup_us = stage_avg_us["gateup"] - spacing
    gateup_s = gateup_us * 1e-6
    gateup_flops = 2.0 * w.P * 2 * w.d * w.f
    traffic = measured_traffic(w.name, mx8, path="stream" if kpath == "stream" else None)
    duration = {"duration_us": gateup_us, "duration_source":
                f"HIP events around the kernel on its launch stream over {args.steps} calls, minus the "
                f"{spacing:.2f} us two back-to-back events measure"}
    traffic_note = ("bytes beyond L2 per launch: FETCH_SIZE + WRITE_SIZE from rocprofv3 counter passes, scaled "
                    "by a plain copy of known size; includes last-level-cache (MALL) hits, so an upper bound of "
                    "the HBM bytes; null once the kernel source changed after the counters were taken")
    if mx8:
        achieved = gateup_flops / gateup_s / 1e12
        roofline = {"bound": "mfma", "kernel": "k_dense<gate/up> (MXFP8 x MXFP4 scaled MFMA)", "achieved": achieved,
                    "peak": MXFP4_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": achieved / MXFP4_PEAK_TFLOPS,
                    "frac_of_fp8_rate": achieved / FP8_PEAK_TFLOPS, "traffic": traffic, "traffic_counter": traffic_note,
                    "algorithmic_flops": gateup_flops, **duration,
                    "peak_note": "the activations are MXFP8, so every product is an FP8 x FP4 scaled MFMA, whose "
                                 "rate is the FP8 one (5.0 PFLOP/s nominal); half the MXFP4 peak (5.05 PFLOP/s) "
                                 "is above that instruction's whole nominal rate and above what it measures here "
                                 "(measured_peak); frac_of_measured is the fraction that bounds this kernel"}
    elif kpath == "stream":
        achieved = gateup_bytes / gateup_s / 1e9
        roofline = {"bound": "hbm", "kernel": "k_expert<gate/up>", "achieved": achieved,
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                    "traffic": traffic, "traffic_counter": traffic_note, "algorithmic_bytes": gateup_bytes,
                    **duration}
    elif "routing in" in kpath:
        # one kernel routes, permutes and runs both projections: all expert
        # bytes, x, the logits and the float32 per-pair outputs it writes
        nbytes = fused_bytes + w.T * w.E * 4
        achieved = nbytes / gateup_s / 1e9
        roofline = {"bound": "hbm", "kernel": "k_layer (routing, permutation, gate/up and down units, one launch)",
                    "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                    "traffic": traffic, "traffic_counter": traffic_note, "algorithmic_bytes": nbytes,
                    **duration}
    else:
        # one kernel runs gate/up and down (the down stage launches nothing)
        achieved = fused_bytes / gateup_s / 1e9
        kname = "k_chain (gate/up and down units, one launch)" if "ticketed" in kpath else \
            "k_fused (persistent: gate/up and down units)"
        roofline = {"bound": "hbm", "kernel": kname, "achieved": achieved,
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                    "traffic": traffic, "traffic_counter": traffic_note, "algorithmic_bytes": fused_bytes,
                    **duration}
    result = {
        "metric": "MoE expert-layer tokens/s + achieved HBM GB/s (% of peak), 256-token verify",
        "value": w.T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": settle,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8xmxfp4" if mx8 else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.T} tokens "
                               f"({'one compute-bound chunk' if mx8 else f'{w.T // 8} sequences x DFlash block 8'}), "
                               f"d_model {w.d}, d_ff {w.f}, {w.E} experts, top-{w.k}, "
                               f"bias {w.bias}, MXFP4 weights (E2M1 + E8M0 per 32), "
                               f"{'MXFP8 (E4M3 + E8M0 per 32)' if mx8 else 'bf16'} activations, bf16 out"
                               f"{', router projection in the call (bf16 W_router [E][d])' if wr is not None else ''}",
                   "T": w.T, "d_model": w.d, "d_ff": w.f, "experts": w.E, "top_k": w.k,
                   "touched_experts": touched, "weight_copies": args.copies, "kernel_path": kpath},
        "layer_hbm_gbs": layer_bytes / (ms_per_step * 1e-3) / 1e9,
        "layer_hbm_frac": layer_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "layer_algorithmic_bytes": layer_bytes,
        "layer_tflops": flops / (ms_per_step * 1e-3) / 1e12,
        "stage_us": stage_avg_us,
        "per_call_ms": pct,
        "roofline": roofline,
    }
    if wr is not None:
        # the projection alone, on torch's current stream, timed with its events
        lgo = torch.empty((w.T, w.E), dtype=torch.float32, device="cuda")
        for _ in range(5):
            layers[0].router_logits(x, wr, out=lgo)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            layers[0].router_logits(x, wr, out=lgo)
        e1.record()
        torch.cuda.synchronize()
        result["router_projection_us"] = e0.elapsed_time(e1) * 1e3 / args.steps
    # the optional legs below report beside the metric; a failure in one is
    # recorded in the line instead of losing it
    if args.graph:
        try:
            result["graph_replay"] = time_graph_replay(layers, x, lg, out, ws, wr, args, torch)
        except Exception as e:                          # noqa: BLE001
            result["graph_replay"] = {"error": repr(e)}
    if args.peaks:
        try:
            peaks = measure_peaks(moe, torch)
            result["measured_peaks"] = peaks
            if roofline["unit"] == "GB/s":
                roofline["measured_peak"] = peaks["stream_read_GBps"]
            else:
                # the rate on operands that toggle like real data; the
                # constant-operand loop runs at a higher clock
                roofline["measured_peak"] = peaks["mfma_fp8xfp4_16x16x128_random"]["TFLOPs"]
                roofline["measured_peak_constant_operands"] = peaks["mfma_fp8xfp4_16x16x128"]["TFLOPs"]
            roofline["frac_of_measured"] = roofline["achieved"] / roofline["measured_peak"]
        except Exception as e:                          # noqa: BLE001
            result["measured_peaks"] = {"error": repr(e)}
    accept_inputs = None
    if args.with_accept and mx8:
        # the 8192-token chunk is a prefill-sized batch, not a verify step
        result["dflash_accept"] = {"skipped": "not a verify batch"}
    elif args.with_accept:
        try:
            result["dflash_accept"], accept_inputs = time_accept(w, args, moe, torch, np, synth)
        except Exception as e:                          # noqa: BLE001
            result["dflash_accept"] = {"error": repr(e)}
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 18                   # float32 elements
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.copy_calibration_mib} MiB read + written, 3 dispatches")
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle on {args.cpu_tokens} tokens")
        rb = synth.router_weights_bf16(w) if wr is not None else None
        result["cpu_baseline"] = cpu_baseline(w, acts, args.cpu_tokens, rb)
        if w.name in ("tiny", "verify_1seq", "verify_32seq") and args.cpu_tokens_1thread > 0:
            n1 = min(args.cpu_tokens_1thread, w.T)
            log(f"timing the CPU oracle on {n1} tokens, one thread")
            result["cpu_baseline_single_thread"] = cpu_baseline(w, acts, n1, rb, threads=1)
        if accept_inputs is not None:
            result["dflash_accept"]["cpu_baseline"] = cpu_baseline_accept(accept_inputs)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
