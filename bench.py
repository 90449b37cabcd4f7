"""Benchmark of the quantized MoE expert layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-prefill]

A step is one pass of the whole layer -- route, quantize x, permute, gate/up
GEMM + SiLU, quantize h, down GEMM, combine -- over one batch of synthetic
input already resident in HBM (at decode the middle three run as the one
fused expert-MLP launch).  The headline workload is the Inkling-Small
sparse layer at decode, T = 4 tokens (256 experts of width 2048, hidden 4096,
top-6, INT4 g128 weights, per-token FP8 activations); its metric is the weight
stream: bytes of the distinct experts' packed weights and scales / step time.
The same run also times the T = 2048 prefill layer (FP8 TFLOP/s and the
fraction of its attainable roofline), the skewed prefill layer with two bf16
shared experts, the row-FP8 layer (384 experts), a supplementary token sweep of
the prefill layer (T = 4096 .. 16384), decode with bf16 group scales and the
NVFP4 + AQLM hybrid decode layer, plus measured copy / read ceilings and the
shader clock before and after.

Weights rotate over several independently generated weight sets so that no
step finds its experts in the 256 MB last-level cache.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer FP8 TFLOP/s at T=2048 prefill; weight-stream GB/s at T=4 decode"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 200 decode steps take ~16 ms: enough that the host-to-device latency of
    # the first launch (paid once per timed region) is a small share of a step
    ap.add_argument("--steps", type=int, default=200)
    # every weight set is read once right after it is built (the first reads of
    # fresh pages are slow); the timed region itself carries a fixed ~50 us (the
    # first launch's host latency and the final synchronize), i.e. ~2.5 us per
    # step at 20 steps and ~0.25 us at 200
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=4, help="weight sets rotated across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-hybrid", action="store_true",
                    help="skip the NVFP4 + AQLM hybrid decode layer")
    ap.add_argument("--no-bf16-scales", action="store_true",
                    help="skip the decode layer with bfloat16 INT4 group scales")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 1 GiB device buffer 5 times (a plain copy kernel of known "
                         "size, to scale the memory-traffic counters), then exit")
    ap.add_argument("--no-graph", action="store_true",
                    help="time only eager launches (default: also replay captured graphs)")
    ap.add_argument("--no-skewed", action="store_true", help="skip the skewed prefill layer")
    ap.add_argument("--no-fp8row", action="store_true", help="skip the row-FP8 prefill layer")
    ap.add_argument("--no-shares", action="store_true",
                    help="skip the single-GPU shares of the expert- and width-sharded layer")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the supplementary prefill token sweep (T = 4096 .. 16384)")
    ap.add_argument("--workload", default="decode", choices=["decode", "prefill", "skewed", "fp8row"])
    ap.add_argument("--tokens", type=int, default=None,
                    help="token count T of the workload (default: the workload's own); for "
                         "profiling one point of the prefill token sweep")
    ap.add_argument("--summarize", metavar="DIR",
                    help="only summarise the rocprofv3 CSV output under DIR (kernel stats, or the "
                         "mean per dispatch of every collected counter per kernel) and exit")
    return ap.parse_args()


def summarize(root: str) -> str:
    """Markdown summary of rocprofv3 CSV output under root: the kernel stats table of
    a --kernel-trace --stats run, or for --pmc runs the mean per dispatch of each
    counter per kernel (libmoeq kernels and the device copy)."""
    import csv
    import glob
    import re

    def short(name):
        name = name.replace("(anonymous namespace)::", "").replace("void ", "")
        name = re.sub(r"\((?!anon).*$", "", name)
        return name.replace("moeq::", "")
    lines = []
    for f in sorted(glob.glob(os.path.join(root, "**", "*kernel_stats.csv"), recursive=True)):
        lines += [f"kernel stats ({os.path.relpath(f, root)})", "",
                  "| kernel | calls | avg us | min us | max us |", "|---|---:|---:|---:|---:|"]
        for r in csv.DictReader(open(f)):
            lines.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
        lines.append("")
    per = {}
    for f in sorted(glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True)):
        for r in csv.DictReader(open(f)):
            k = short(r.get("Kernel_Name", ""))
            if not (k.split("<")[0].endswith("kernel") or "copyBuffer" in k):
                continue
            per.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if per:
        lines += ["| kernel | counter | dispatches | mean per dispatch |", "|---|---|---:|---:|"]
        for k in sorted(per):
            for c in sorted(per[k]):
                v = per[k][c]
                lines.append(f"| `{k}` | {c} | {len(v)} | {sum(v) / len(v):.1f} |")
    return "\n".join(lines)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def expert_bytes(cfg) -> tuple:
    """Algorithmic bytes of one expert's weights: (w13, w2) incl. scales."""
    if cfg.weight_format in ("w4a8", "w4a8_bf16s"):
        sb = 2 if cfg.weight_format == "w4a8_bf16s" else 4      # bytes per group scale
        w13 = 2 * cfg.I * cfg.H // 2 + 2 * cfg.I * (cfg.H // 128) * sb
        w2 = cfg.H * cfg.I // 2 + cfg.H * (cfg.I // 128) * sb
    else:
        w13 = 2 * cfg.I * cfg.H + 2 * cfg.I * 4
        w2 = cfg.H * cfg.I + cfg.H * 4
    return w13, w2


def build_sets(cfg, n_sets, dev):
    import dataclasses

    import torch

    import bit_quantized_moe_top_amd as mq
    import workloads as W
    layers = []
    for s in range(n_sets):
        c = dataclasses.replace(cfg, seed=cfg.seed + 1000 * s)
        layer = mq.MoELayer(c.H, c.I, c.E, c.k, c.weight_format, device=dev)
        fp8 = c.weight_format == "fp8row"
        # E4M3 rows, or INT4 in the GEMMs' tiled order [E, N/16, K/128, 16, 64]
        w13 = torch.empty((c.E, 2 * c.I, c.H) if fp8 else (c.E, 2 * c.I // 16, c.H // 128, 16, 64),
                          dtype=torch.uint8, device=dev)
        w2 = torch.empty((c.E, c.H, c.I) if fp8 else (c.E, c.H // 16, c.I // 128, 16, 64),
                         dtype=torch.uint8, device=dev)
        sdt = torch.bfloat16 if c.weight_format == "w4a8_bf16s" else torch.float32
        s13 = torch.empty((c.E, 2 * c.I) if fp8 else (c.E, 2 * c.I, c.H // 128), dtype=sdt,
                          device=dev)
        s2 = torch.empty((c.E, c.H) if fp8 else (c.E, c.H, c.I // 128), dtype=sdt, device=dev)
        quant = mq.quant_fp8_per_token if fp8 else \
            (lambda wf, wq, ws: mq.pack_int4_g128(wf, wq, ws, tiled=True))
        for which, wq, ws in (("w13", w13, s13), ("w2", w2, s2)):
            for e0, wf in W.iter_expert_weights(c, which, dev, chunk=32):
                quant(wf, wq[e0:e0 + wf.shape[0]], ws[e0:e0 + wf.shape[0]])
                del wf
        layer.set_weights(w13, s13, w2, s2)
        if c.n_shared:
            layer.set_shared(*W.make_shared_weights(c, dev))
        inp = W.make_layer_inputs(c, device=dev, weights=False)
        layers.append((layer, inp))
        touch(layer.w13, layer.s13, layer.w2, layer.s2, layer.ws13, layer.ws2)
        torch.cuda.synchronize()
        log(f"{cfg.name}: weight set {s + 1}/{n_sets} ready")
    return layers


def touch(*tensors):
    """Reads every byte of the given tensors once (untimed): the first reads of
    freshly written weight pages are slower than later ones."""
    import torch
    for t in tensors:
        if t is not None:
            torch.sum(t.view(torch.uint8), dtype=torch.int64)


SETTLE_S = 0.2


def settle(run, n_sets, seconds=SETTLE_S):
    """Untimed: runs the step function run(i) for about `seconds`, in chunks of 50
    steps between synchronizations, before the W warm-up steps.  Over the first
    tenths of a second of sustained work the clocks ramp up and per-step times
    fall (measured at T = 4: 68.0 us per step over the first 200 steps, 66.1 us
    over 2000), so a short timed region taken right after weight generation
    would depend on how long the warm-up is."""
    import torch
    t_end = time.perf_counter() + seconds
    i = 0
    while time.perf_counter() < t_end:
        for _ in range(50):
            run(i % n_sets)
            i += 1
        torch.cuda.synchronize()


def time_layer(cfg, n_sets, steps, warmup, dev, graph=False, split_events=False, layers=None):
    """Times `steps` layer passes; returns timings and the per-call launch times
    (with split_events the expert MLP's three calls are timed one by one).
    layers: already built (layer, inputs) pairs to time instead of new weight sets."""
    import torch

    import bit_quantized_moe_top_amd as mq
    if layers is None:
        layers = build_sets(cfg, n_sets, dev)
    n_sets = len(layers)
    # distinct experts touched per set (bytes the step must stream)
    distinct = []
    for layer, inp in layers:
        ids, _ = mq.moe_route_topk(inp["logits"], cfg.k, inp["bias"])
        distinct.append(len(torch.unique(ids)))
    torch.cuda.synchronize()

    # Settle, warm up, then time `steps` whole-layer passes (wall clock between
    # device synchronizations) and, in a second identical pass, each call's launch
    # duration with events on the stream it runs on (the current torch stream).
    def run(i):
        layer, inp = layers[i]
        layer.forward(inp["x"], inp["logits"], inp["bias"])
    settle(run, n_sets)
    for i in range(warmup):
        layer, inp = layers[i % n_sets]
        layer.forward(inp["x"], inp["logits"], inp["bias"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        layer, inp = layers[i % n_sets]
        layer.forward(inp["x"], inp["logits"], inp["bias"])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    graph_ms = None
    if graph:
        # the same steps replayed from one captured graph per weight set (the
        # launches of a step, recorded once; no host work per launch)
        graphs = []
        for layer, inp in layers:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                layer.forward(inp["x"], inp["logits"], inp["bias"])
            graphs.append(g)
        for i in range(warmup):
            graphs[i % n_sets].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            graphs[i % n_sets].replay()
        torch.cuda.synchronize()
        graph_ms = 1e3 * (time.perf_counter() - t0) / steps
        del graphs
    def call_times(split):
        ev = []
        for i in range(steps):
            layer, inp = layers[i % n_sets]
            layer.forward(inp["x"], inp["logits"], inp["bias"], events=ev, split_mlp=split)
        torch.cuda.synchronize()
        per_call = {}
        for name, s, e in ev:
            per_call.setdefault(name, []).append(s.elapsed_time(e))
        # medians: one stalled call (a rare host or device hiccup) must not
        # stand for the call's duration
        return {k: 1e3 * sorted(v)[len(v) // 2] for k, v in per_call.items()}

    per_call_us = call_times(split_events)
    # the expert MLP's calls one by one (its gate/up launch is the layer's dominant kernel)
    split_us = per_call_us if split_events else call_times(True)
    # The dominant kernel alone: `steps` back-to-back gate/up launches over the
    # rotated weight sets (each with the plan and activations of its own last
    # forward), between one pair of events on the launch stream -- the average
    # launch duration without the per-call event overhead.
    import bit_quantized_moe_top_amd as mq
    T = layers[0][1]["x"].shape[0]
    for layer, inp in layers:
        layer.forward(inp["x"], inp["logits"], inp["bias"])

    def gate_up(i):
        layer = layers[i % n_sets][0]
        b = layer.buffers(T)
        gemm = mq.moe_grouped_gemm_fp8row if layer.weight_format == "fp8row" \
            else mq.moe_grouped_gemm_w4a8
        gemm(b["xp_q"], b["xp_s"], b["plan"], layer.w13, layer.s13, epilogue=mq.EPI_SILU_MUL,
             out=b["h"])
    for i in range(warmup):
        gate_up(i)
    # one event pair per launch (the launch's own duration: the host issues the
    # launches faster than the device runs them, so no host time falls inside a
    # pair) and one pair around all of them (the period, with the gaps between
    # consecutive launches)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s_ev.record()
    for i in range(steps):
        evs[i][0].record()
        gate_up(i)
        evs[i][1].record()
    e_ev.record()
    torch.cuda.synchronize()
    gate_up_period_us = 1e3 * s_ev.elapsed_time(e_ev) / steps
    gate_up_us = 1e3 * sum(a.elapsed_time(b) for a, b in evs) / steps
    steps_distinct = [distinct[i % n_sets] for i in range(steps)]
    return {"wall_s": wall, "ms_per_step": 1e3 * wall / steps,
            "graph_ms_per_step": graph_ms,
            "per_call_us": per_call_us, "split_call_us": split_us,
            "gate_up_back_to_back_us": gate_up_us, "gate_up_period_us": gate_up_period_us,
            "distinct_mean": sum(steps_distinct) / steps, "distinct_per_set": distinct,
            "layers": layers}


def time_hybrid(cfg, n_sets, steps, warmup, dev):
    """The NVFP4 + AQLM hybrid layer (hot NVFP4 slabs, cold AQLM slabs): wall time
    per step over `steps` passes rotating `n_sets` independently drawn layers,
    per-call times, and the algorithmic bytes each step streams."""
    import dataclasses

    import torch

    import bit_quantized_moe_top_amd as mq
    import workloads as W
    layers = []
    for s in range(n_sets):
        c = dataclasses.replace(cfg, seed=cfg.seed + 1000 * s)
        hot, cold = W.hybrid_partition(c)
        layer = mq.HybridMoELayer(c.H, c.I, c.E, c.k, device=dev)
        layer.set_hybrid_weights(hot, cold, W.make_nvfp4_slabs(c, len(hot), dev),
                                 W.make_aqlm_slabs(c, len(cold), dev))
        inp = W.make_layer_inputs(c, device=dev, weights=False)
        layers.append((layer, inp, set(hot.tolist())))
        for part in (layer.hot, layer.cold):
            for v in part.values():
                touch(*(v if isinstance(v, list) else [v]))
        torch.cuda.synchronize()
        log(f"{cfg.name}: weight set {s + 1}/{n_sets} ready")
    # bytes per expert: hot = E2M1 codes + E4M3 block scales (+ scale2); cold = the
    # code tensors of every book + fp16 row scales; the codebooks once per step
    H, I = cfg.H, cfg.I
    hot_b = (2 * I * H // 2 + 2 * I * H // 16 + 4) + (H * I // 2 + H * I // 16 + 4)
    cold_b = sum((2 * I * H // 8) * (2 if n > 256 else 1) for n in W.AQLM_BOOKS["w13"]) + \
        2 * I * 2 + sum((H * I // 8) * (2 if n > 256 else 1) for n in W.AQLM_BOOKS["w2"]) + H * 2
    book_b = 16 * (sum(W.AQLM_BOOKS["w13"]) + sum(W.AQLM_BOOKS["w2"]))
    step_bytes, n_hot_touched = [], []
    for layer, inp, hot in layers:
        ids, _ = mq.moe_route_topk(inp["logits"], cfg.k, inp["bias"])
        touched = set(torch.unique(ids).tolist())
        nh = len(touched & hot)
        n_hot_touched.append(nh)
        step_bytes.append(nh * hot_b + (len(touched) - nh) * cold_b + book_b)

    def run(i):
        layer, inp, _ = layers[i]
        layer.forward(inp["x"], inp["logits"], inp["bias"])
    settle(run, n_sets)
    for i in range(warmup):
        layer, inp, _ = layers[i % n_sets]
        layer.forward(inp["x"], inp["logits"], inp["bias"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        layer, inp, _ = layers[i % n_sets]
        layer.forward(inp["x"], inp["logits"], inp["bias"])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = []
    for i in range(steps):
        layer, inp, _ = layers[i % n_sets]
        layer.forward(inp["x"], inp["logits"], inp["bias"], events=ev)
    torch.cuda.synchronize()
    per_call = {}
    for name, s_, e_ in ev:
        per_call.setdefault(name, []).append(s_.elapsed_time(e_))
    del layers
    ms = 1e3 * wall / steps
    mean_bytes = sum(step_bytes[i % n_sets] for i in range(steps)) / steps
    return {"ms_per_step": ms, "bytes_per_step": mean_bytes,
            "hot_experts_touched": sum(n_hot_touched) / n_sets,
            "per_call_us": {k: 1e3 * sorted(v)[len(v) // 2] for k, v in per_call.items()}}


def measured_traffic(kernel_bytes: float, name: str = "gemm_gate_up_decode_T4_traffic"):
    """HBM bytes per launch of a layer's gate/up GEMM from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary profiles/<name>.json, if the
    kernel sources are still the ones the counters were taken on (else None),
    with the down GEMM's and the summary's matrix-core counters when it has them."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name + ".json")
    try:
        doc = json.load(open(path))
        h = hashlib.sha256()
        for f in doc["sources"]:
            h.update(open(os.path.join(ROOT, "bit_quantized_moe_top_amd", "csrc", f), "rb").read())
        if h.hexdigest() != doc["source_sha256"]:
            return None
        out = {"bytes_per_launch": doc["hbm_bytes_per_launch"],
               "vs_algorithmic": round(doc["hbm_bytes_per_launch"] / kernel_bytes, 4),
               "source": f"profiles/{name}.md"}
        if "down_gemm" in doc:
            out["down_bytes_per_launch"] = doc["down_gemm"]["hbm_bytes_per_launch"]
        if "mfma" in doc:
            out["mfma"] = doc["mfma"]
        return out
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(cfg, layers, target_s=10.0):
    """The oracle, as it stands, on the host: full layer for the first weight set."""
    import numpy as np
    import torch

    import workloads as W
    from oracle import formats as F
    from oracle import layer as L
    layer, inp = layers[0]
    x = inp["x"].float().cpu().numpy()
    lg = inp["logits"].cpu().numpy()
    bias = None if inp["bias"] is None else inp["bias"].cpu().numpy()
    ids, _ = L.route_topk(lg, cfg.k, bias)
    experts = sorted(set(ids.reshape(-1).tolist()))
    import dataclasses
    c = dataclasses.replace(cfg, seed=cfg.seed)       # set 0 uses the base seed
    packed13, sc13, packed2, sc2 = {}, {}, {}, {}
    for e in experts:                                  # weight preparation: not timed
        packed13[e], sc13[e] = L.pack_int4_g128(W.expert_weight(c, "w13", e, inp["x"].device).cpu().numpy())
        packed2[e], sc2[e] = L.pack_int4_g128(W.expert_weight(c, "w2", e, inp["x"].device).cpu().numpy())
    reps, t_total = 0, 0.0
    while t_total < target_s and reps < 20:
        t0 = time.perf_counter()
        L.moe_layer(x, lg, cfg.k, bias=bias, packed13=packed13, scales13=sc13, packed2=packed2,
                    scales2=sc2)
        t_total += time.perf_counter() - t0
        reps += 1
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas = 1
    sec = t_total / reps
    w13b, w2b = expert_bytes(cfg)
    gbs = len(experts) * (w13b + w2b) / sec / 1e9
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    _ = (np, torch, F)
    return {"value": gbs, "unit": "GB/s", "cores": blas, "kind": "oracle",
            "sample": f"the full decode layer (T={cfg.T}, {len(experts)} distinct experts) "
                      f"route->combine on oracle-prepacked weights, mean of {reps} runs "
                      f"({sec:.2f} s each); host CPU {cpu}; BLAS threads {blas}, "
                      f"elementwise NumPy single-threaded",
            "seconds_per_layer": sec}


def prefill_summary(pcfg, pres, short=False):
    """FP8 TFLOP/s of a T-token layer and its fractions of the FP8 peak and of
    the attainable roofline min(peak FLOP/s, HBM bandwidth x arithmetic intensity)."""
    pms = pres["ms_per_step"]
    t = pms * 1e-3
    fp8_flops = 2.0 * pcfg.R * 3 * pcfg.H * pcfg.I
    pw13, pw2 = expert_bytes(pcfg)
    wbytes = pres["distinct_mean"] * (pw13 + pw2)
    S = pcfg.n_shared * pcfg.I
    bf16_flops = 2.0 * pcfg.T * 3 * pcfg.H * S
    shared_bytes = 3 * pcfg.H * S * 2
    io_bytes = pcfg.T * pcfg.H * 2 * 2 + pcfg.T * pcfg.E * 4       # x in, y out, logits
    total_bytes = wbytes + shared_bytes + io_bytes
    t_roof = max(total_bytes / (HBM_PEAK_GBS * 1e9),
                 fp8_flops / (FP8_PEAK_TFLOPS * 1e12) + bf16_flops / (BF16_PEAK_TFLOPS * 1e12))
    fmt = {"w4a8": "INT4 g128", "w4a8_bf16s": "INT4 g128 (bf16 scales)", "fp8row": "row FP8"}
    d = {"workload": f"{pcfg.name}: T={pcfg.T}, hidden {pcfg.H}, {pcfg.E} experts of width "
                     f"{pcfg.I}, top-{pcfg.k}, {fmt.get(pcfg.weight_format, pcfg.weight_format)}"
                     + (f", {pcfg.n_shared} bf16 shared experts" if pcfg.n_shared else ""),
         "T": pcfg.T,
         "value": round(fp8_flops / t / 1e12, 2), "unit": "TFLOP/s",
         "ms_per_step": round(pms, 4),
         "frac_fp8_peak": round(fp8_flops / t / 1e12 / FP8_PEAK_TFLOPS, 4),
         "roofline_us": round(t_roof * 1e6, 1),
         "frac_attainable_roofline": round(t_roof / t, 4),
         "bytes_per_step": round(total_bytes),
         "hbm_GBps": round(total_bytes / t / 1e9, 1),
         "gate_up_gemm_us": round(pres["gate_up_back_to_back_us"], 2),
         "gate_up_gemm_GBps": round(pres["distinct_mean"] * pw13 /
                                    (pres["gate_up_back_to_back_us"] * 1e-6) / 1e9, 1),
         "per_call_us": {k: round(v, 2) for k, v in pres["per_call_us"].items()}}
    pc = pres["per_call_us"]
    if "gemm_down" in pc:
        d["down_gemm_GBps"] = round(pres["distinct_mean"] * pw2 / (pc["gemm_down"] * 1e-6) / 1e9, 1)
    if not short:
        tr = measured_traffic(pres["distinct_mean"] * pw13,
                              f"gemm_gate_up_{pcfg.name}_T{pcfg.T}_traffic")
        if tr is not None:
            d["gate_up_traffic"] = tr
    if pcfg.n_shared:
        sh_us = pc.get("shared_gate_up", 0.0) + pc.get("shared_down", 0.0)
        d["shared_bf16"] = {"flops": bf16_flops, "us": round(sh_us, 2),
                            "TFLOPs": round(bf16_flops / (sh_us * 1e-6) / 1e12, 1) if sh_us else None,
                            "frac_bf16_peak": round(bf16_flops / (sh_us * 1e-6) / 1e12 /
                                                    BF16_PEAK_TFLOPS, 4) if sh_us else None}
    if short:
        for k in ("workload", "per_call_us", "bytes_per_step"):
            d.pop(k)
    return d


def torch_shared_gemm_us(cfg, dev, reps=20):
    """Beside the library's shared-expert GEMMs: torch.matmul (ROCm's BLAS) on
    the same bf16 shapes, gate/up [T, H] x [H, 2S] and down [T, S] x [S, H]
    (products only, no SiLU), median microseconds per call."""
    import torch
    S = cfg.n_shared * cfg.I
    g = torch.Generator(device=dev).manual_seed(cfg.seed)
    out = {}
    for name, (m, k, n) in (("gate_up", (cfg.T, cfg.H, 2 * S)), ("down", (cfg.T, S, cfg.H))):
        a = torch.randn(m, k, device=dev, generator=g).to(torch.bfloat16)
        w = (torch.randn(n, k, device=dev, generator=g) * 0.05).to(torch.bfloat16)
        wt = w.t()
        for _ in range(3):
            torch.matmul(a, wt)
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            torch.matmul(a, wt)
            e1.record()
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
        out[name] = round(sorted(times)[reps // 2], 2)
    return out


def copy_ceiling(dev, nbytes=2 << 30, reps=5):
    """Measured streaming ceilings on this machine: a device-to-device copy of nbytes
    with torch's copy kernel (bytes read + written per second), and the library's
    streaming-read probe over nbytes at a time, rotating through four such chunks
    so that no chunk is still in the 256 MB last-level cache (bytes read per
    second)."""
    import torch

    import bit_quantized_moe_top_amd as mq
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    big = torch.ones(4 * nbytes // 4, dtype=torch.float32, device=dev)
    chunks = [big[i * (nbytes // 4):(i + 1) * (nbytes // 4)] for i in range(4)]
    sink = torch.empty(mq.READ_PROBE_BLOCKS * 4, dtype=torch.int32, device=dev)
    probe_i = [0]

    def probe():
        mq.moe_read_bandwidth_probe(chunks[probe_i[0] % 4], sink)
        probe_i[0] += 1

    def timed(fn):
        fn()
        s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_ev.record()
        for _ in range(reps):
            fn()
        e_ev.record()
        torch.cuda.synchronize()
        return s_ev.elapsed_time(e_ev) * 1e-3 / reps
    copy_s = timed(lambda: dst.copy_(src))
    read_s = timed(probe)
    del src, dst, big, chunks
    torch.cuda.empty_cache()
    return {"GBps": round(2 * nbytes / copy_s / 1e9, 1), "bytes": nbytes,
            "kind": "device copy (read + write), torch copy kernel",
            "read_GBps": round(nbytes / read_s / 1e9, 1),
            "read_kind": f"moe_read_bandwidth_probe over {nbytes >> 30} GiB at a time, four "
                         f"chunks in rotation (bytes read)"}


def sclk_mhz():
    """Current shader clock (MHz) of the GPU(s) from the amdgpu kernel driver's DPM table, if readable."""
    import glob
    vals = []
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(path):
                if line.strip().endswith("*"):
                    vals.append(int(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0]))
        except (OSError, ValueError, IndexError):
            pass
    return vals or None


def main():
    args = parse()
    if args.summarize:
        print(summarize(args.summarize))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the layer would shard by experts or by width across GPUs; this library "
              f"runs on one GPU).", file=sys.stderr)
        sys.exit(2)
    import torch

    import workloads as W
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)      # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "copies": 5}))
        return
    cfg = W.get_config(args.workload, **({"T": args.tokens} if args.tokens else {}))
    log(f"device {torch.cuda.get_device_name(0)}; workload {cfg}")
    sclk_before = sclk_mhz()
    res = time_layer(cfg, args.sets, args.steps, args.warmup, dev, graph=not args.no_graph,
                     split_events=cfg.R > 64)
    w13b, w2b = expert_bytes(cfg)
    D = res["distinct_mean"]
    flops = 2.0 * cfg.R * 3 * cfg.H * cfg.I
    # headline: the faster of eager launches and graph replay (both reported)
    ms_eager = res["ms_per_step"]
    ms_graph = res["graph_ms_per_step"]
    ms = min(ms_eager, ms_graph) if ms_graph else ms_eager
    gbs = D * (w13b + w2b) / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    # the dominant kernel: the gate/up grouped GEMM (SiLU epilogue), the first
    # launch of the expert MLP; its average launch duration from back-to-back
    # launches bracketed by one pair of events
    dom_name = "moe_grouped_gemm gate/up (SiLU epilogue; first launch of moe_expert_mlp)"
    dom_bytes = D * w13b
    dom_us = res["gate_up_back_to_back_us"]
    dom_gbs = dom_bytes / (dom_us * 1e-6) / 1e9
    traffic = measured_traffic(dom_bytes) if cfg.name == "decode" else None
    out = {
        "metric": METRIC,
        "value": round(gbs if cfg.name == "decode" else tflops, 3),
        "unit": "GB/s" if cfg.name == "decode" else "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle_s": SETTLE_S,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3 x int4->e4m3, fp32 accumulate",
        "data": "synthetic (seeded; random-init weights of the Inkling-Small expert shapes)",
        "config": {"workload": f"{cfg.name}: T={cfg.T} tokens, hidden {cfg.H}, {cfg.E} experts of "
                               f"width {cfg.I}, top-{cfg.k}, "
                               f"{'INT4 g128' if cfg.weight_format == 'w4a8' else 'row FP8'} "
                               f"weights, per-token FP8 activations, bf16 out",
                   "distinct_experts_per_step": D, "weight_sets_rotated": args.sets,
                   "flops_per_step": flops,
                   "weight_bytes_per_step": D * (w13b + w2b)},
        "roofline": {"kernel": dom_name, "bound": "hbm",
                     "achieved": round(dom_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                     "traffic": (traffic or {}).get("bytes_per_launch"),
                     "traffic_detail": traffic,
                     "avg_launch_us": round(dom_us, 3),
                     "launch_period_us": round(res["gate_up_period_us"], 3),
                     "timing": "an event pair around each of `steps` back-to-back launches on the "
                               "launch stream (launch_period_us: one pair around all of them, "
                               "with the gaps between launches)",
                     "bytes_per_launch": dom_bytes},
        "layer_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "launch_mode": "hip graph replay" if ms_graph and ms_graph <= ms_eager else "eager",
        "eager_ms_per_step": round(ms_eager, 5),
        "graph_ms_per_step": round(ms_graph, 5) if ms_graph else None,
        "per_call_us": {k: round(v, 2) for k, v in res["per_call_us"].items()},
        "expert_mlp_split_call_us": {k: round(v, 2) for k, v in res["split_call_us"].items()
                                     if k in ("gemm_gate_up", "quant_h", "gemm_down")},
    }
    layers = res.pop("layers")
    if not args.no_cpu_baseline and cfg.name == "decode":
        log("timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(cfg, layers)
    del layers
    torch.cuda.empty_cache()
    if not args.no_prefill and cfg.name == "decode":
        pcfg = W.get_config("prefill")
        psteps = max(5, args.steps // 2)
        pres = time_layer(pcfg, 2, psteps, 2, dev, split_events=True)
        out["prefill"] = prefill_summary(pcfg, pres)
        if not args.no_sweep:
            # supplementary: the same layer (weight set 0) at larger token counts,
            # where the grouped GEMMs have enough rows per expert to become
            # MFMA-bound; not one of the named workloads
            layer = pres["layers"][0][0]
            sweep = []
            for T in (4096, 8192, 16384):
                scfg = W.get_config("prefill", T=T)
                sres = time_layer(scfg, 1, 5, 2, dev, split_events=True,
                                  layers=[(layer, W.make_layer_inputs(scfg, dev, weights=False))])
                sres.pop("layers")
                sweep.append(prefill_summary(scfg, sres, short=True))
                layer._bufs.clear()
                torch.cuda.empty_cache()
            out["t_sweep"] = {"note": "supplementary prefill token sweep of the prefill layer "
                                      "(not one of the named workloads)", "points": sweep}
        pres.pop("layers")
        torch.cuda.empty_cache()
    for name, skip in (("skewed", args.no_skewed), ("fp8row", args.no_fp8row)):
        if skip or cfg.name != "decode" or args.no_prefill:
            continue
        scfg = W.get_config(name)
        sres = time_layer(scfg, 2, max(5, args.steps // 2), 2, dev, split_events=True)
        sres.pop("layers")
        out[name] = prefill_summary(scfg, sres)
        if scfg.n_shared:
            out[name]["shared_bf16"]["torch_matmul_us"] = torch_shared_gemm_us(scfg, dev)
        torch.cuda.empty_cache()
    if not args.no_shares and not args.no_prefill and cfg.name == "decode":
        import dataclasses
        # supplementary: what one GPU runs when the layer is sharded over eight
        # (not one of the named workloads; no collective is timed)
        shares = {"note": "one GPU's share of the layer sharded over 8 GPUs: EP8 holds 32 of the "
                          "256 experts and receives 1/8 of the routed rows (T = 2048 -> 1536 rows); "
                          "TP8 holds 1/8 of every expert's width (w13 512 rows, w2 K = 256)"}
        for name, base, over in (("ep8_prefill", "prefill", {"E": 32, "T": 256}),
                                 ("tp8_prefill", "prefill", {"I": 256}),
                                 ("tp8_decode", "decode", {"I": 256})):
            scfg = dataclasses.replace(W.get_config(base, **over), name=name)
            sres = time_layer(scfg, 2 if base == "prefill" else args.sets, max(5, args.steps // 2),
                              2 if base == "prefill" else args.warmup, dev,
                              split_events=scfg.R > 64)
            sres.pop("layers")
            if base == "prefill":
                shares[name] = prefill_summary(scfg, sres, short=True)
            else:
                sw13, sw2 = expert_bytes(scfg)
                sms = sres["ms_per_step"]
                shares[name] = {"ms_per_step": round(sms, 5),
                                "weight_bytes_per_step": sres["distinct_mean"] * (sw13 + sw2),
                                "value": round(sres["distinct_mean"] * (sw13 + sw2) / (sms * 1e-3)
                                               / 1e9, 1), "unit": "GB/s",
                                "gate_up_gemm_us": round(sres["gate_up_back_to_back_us"], 2),
                                "per_call_us": {k: round(v, 2)
                                                for k, v in sres["per_call_us"].items()}}
            torch.cuda.empty_cache()
        out["shard_shares"] = shares
    if not args.no_bf16_scales and cfg.name == "decode":
        import dataclasses
        bcfg = dataclasses.replace(cfg, weight_format="w4a8_bf16s")
        bres = time_layer(bcfg, args.sets, args.steps, args.warmup, dev, graph=False)
        bres.pop("layers")
        bw13, bw2 = expert_bytes(bcfg)
        bms = bres["ms_per_step"]
        out["decode_bf16_scales"] = {
            "workload": "decode as above with bfloat16 INT4 group scales (the 16-bit scales of "
                        "the W4A8 checkpoint)",
            "ms_per_step": round(bms, 5),
            "weight_bytes_per_step": bres["distinct_mean"] * (bw13 + bw2),
            "value": round(bres["distinct_mean"] * (bw13 + bw2) / (bms * 1e-3) / 1e9, 1),
            "unit": "GB/s",
            "gate_up_gemm_us": round(bres["gate_up_back_to_back_us"], 2),
            "per_call_us": {k: round(v, 2) for k, v in bres["per_call_us"].items()},
        }
        torch.cuda.empty_cache()
    if not args.no_hybrid and cfg.name == "decode":
        hcfg = W.get_config("hybrid_decode")
        hres = time_hybrid(hcfg, args.sets, args.steps, args.warmup, dev)
        hms = hres["ms_per_step"]
        out["hybrid_decode"] = {
            "workload": f"NVFP4 + AQLM hybrid decode: T={hcfg.T}, hidden {hcfg.H}, {hcfg.E} "
                        f"experts of width {hcfg.I}, top-{hcfg.k}, "
                        f"{round(W.HYBRID_HOT_FRACTION * 100, 1)}% hot (NVFP4), cold AQLM 2-bit "
                        f"(w13 one 65536-entry book, w2 65536 + 256)",
            "ms_per_step": round(hms, 5),
            "weight_bytes_per_step": round(hres["bytes_per_step"]),
            "hot_experts_touched_per_step": hres["hot_experts_touched"],
            "value": round(hres["bytes_per_step"] / (hms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "per_call_us": {k: round(v, 2) for k, v in hres["per_call_us"].items()},
        }
        torch.cuda.empty_cache()
    out["copy_ceiling"] = copy_ceiling(dev)
    ceil_gbs = out["copy_ceiling"]["read_GBps"]
    out["layer_frac_of_read_ceiling"] = round(gbs / ceil_gbs, 4) if cfg.name == "decode" else None
    # the dominant kernel and the prefill GEMMs against the measured read ceiling
    # (the roofline's peak stays the interface's published 8 TB/s)
    out["roofline"]["read_ceiling_GBps"] = ceil_gbs
    out["roofline"]["frac_of_read_ceiling"] = round(dom_gbs / ceil_gbs, 4)
    for name in ("prefill", "skewed", "fp8row"):
        if name in out:
            for key in ("gate_up_gemm_GBps", "down_gemm_GBps"):
                if key in out[name]:
                    out[name][key.replace("_GBps", "_frac_of_read_ceiling")] = \
                        round(out[name][key] / ceil_gbs, 4)
    out["sclk_mhz"] = {"before": sclk_before, "after": sclk_mhz()}
    out["host"] = platform.node()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
