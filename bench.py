"""Benchmark of the quantized MoE expert layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-prefill]

A step is one pass of the whole layer -- route, quantize x, permute, gate/up
GEMM + SiLU, quantize h, down GEMM, combine -- over one batch of synthetic
input already resident in HBM (at decode the middle three run as the one
fused expert-MLP launch).  The headline workload is the Inkling-Small
sparse layer at decode, T = 4 tokens (256 experts of width 2048, hidden 4096,
top-6, INT4 g128 weights, per-token FP8 activations); its metric is the weight
stream: bytes of the distinct experts' packed weights and scales / step time.
The same run also times the T = 2048 prefill layer and reports its FP8 TFLOP/s.

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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 200 decode steps take ~16 ms: enough that the host-to-device latency of
    # the first launch (paid once per timed region) is a small share of a step
    ap.add_argument("--steps", type=int, default=200)
    # the first ~200 decode steps after the weight sets are built run ~5% slower
    # than the steady state (first touches of the weight pages), so the default
    # warm-up covers them; the timed steps are the same with any warm-up
    ap.add_argument("--warmup", type=int, default=200)
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
    ap.add_argument("--workload", default="decode", choices=["decode", "prefill", "skewed", "fp8row"])
    return ap.parse_args()


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
        kd13, kd2 = (c.H, c.I) if fp8 else (c.H // 2, c.I // 2)
        w13 = torch.empty(c.E, 2 * c.I, kd13, dtype=torch.uint8, device=dev)
        w2 = torch.empty(c.E, c.H, kd2, dtype=torch.uint8, device=dev)
        sdt = torch.bfloat16 if c.weight_format == "w4a8_bf16s" else torch.float32
        s13 = torch.empty((c.E, 2 * c.I) if fp8 else (c.E, 2 * c.I, c.H // 128), dtype=sdt,
                          device=dev)
        s2 = torch.empty((c.E, c.H) if fp8 else (c.E, c.H, c.I // 128), dtype=sdt, device=dev)
        quant = mq.quant_fp8_per_token if fp8 else mq.pack_int4_g128
        for which, wq, ws in (("w13", w13, s13), ("w2", w2, s2)):
            for e0, wf in W.iter_expert_weights(c, which, dev, chunk=32):
                quant(wf, wq[e0:e0 + wf.shape[0]], ws[e0:e0 + wf.shape[0]])
                del wf
        layer.set_weights(w13, s13, w2, s2)
        if c.n_shared:
            layer.set_shared(*W.make_shared_weights(c, dev))
        inp = W.make_layer_inputs(c, device=dev, weights=False)
        layers.append((layer, inp))
        torch.cuda.synchronize()
        log(f"{cfg.name}: weight set {s + 1}/{n_sets} ready")
    return layers


def time_layer(cfg, n_sets, steps, warmup, dev, graph=False, split_events=False):
    """Times `steps` layer passes; returns timings and the per-call launch times
    (with split_events the expert MLP's three calls are timed one by one)."""
    import torch

    import bit_quantized_moe_top_amd as mq
    layers = build_sets(cfg, n_sets, dev)
    # distinct experts touched per set (bytes the step must stream)
    distinct = []
    for layer, inp in layers:
        ids, _ = mq.moe_route_topk(inp["logits"], cfg.k, inp["bias"])
        distinct.append(len(torch.unique(ids)))
    torch.cuda.synchronize()

    # Warm up, then time `steps` whole-layer passes (wall clock between device
    # synchronizations) and, in a second identical pass, each call's launch
    # duration with events on the stream it runs on (the current torch stream).
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
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s_ev.record()
    for i in range(steps):
        gate_up(i)
    e_ev.record()
    torch.cuda.synchronize()
    gate_up_us = 1e3 * s_ev.elapsed_time(e_ev) / steps
    steps_distinct = [distinct[i % n_sets] for i in range(steps)]
    return {"wall_s": wall, "ms_per_step": 1e3 * wall / steps,
            "graph_ms_per_step": graph_ms,
            "per_call_us": per_call_us, "split_call_us": split_us,
            "gate_up_back_to_back_us": gate_up_us,
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
    """HBM bytes per launch of the decode layer's dominant kernel from the
    committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, if the kernel sources
    are still the ones the counters were taken on (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name + ".json")
    try:
        doc = json.load(open(path))
        h = hashlib.sha256()
        for f in doc["sources"]:
            h.update(open(os.path.join(ROOT, "bit_quantized_moe_top_amd", "csrc", f), "rb").read())
        if h.hexdigest() != doc["source_sha256"]:
            return None
        return {"bytes_per_launch": doc["hbm_bytes_per_launch"],
                "vs_algorithmic": round(doc["hbm_bytes_per_launch"] / kernel_bytes, 4),
                "source": f"profiles/{name}.md"}
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


def main():
    args = parse()
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
    cfg = W.get_config(args.workload)
    log(f"device {torch.cuda.get_device_name(0)}; workload {cfg}")
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
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
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
                     "timing": "events around back-to-back launches on the launch stream",
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
        pres = time_layer(pcfg, 2, max(5, args.steps // 2), 2, dev, split_events=True)
        pms = pres["ms_per_step"]
        pflops = 2.0 * pcfg.R * 3 * pcfg.H * pcfg.I
        ptf = pflops / (pms * 1e-3) / 1e12
        pw13, pw2 = expert_bytes(pcfg)
        pbytes = pres["distinct_mean"] * (pw13 + pw2)
        t_roof = max(pbytes / (HBM_PEAK_GBS * 1e9), pflops / (FP8_PEAK_TFLOPS * 1e12))
        out["prefill"] = {
            "workload": f"prefill: T={pcfg.T}, hidden {pcfg.H}, {pcfg.E} experts of width {pcfg.I}, "
                        f"top-{pcfg.k}, INT4 g128",
            "value": round(ptf, 2), "unit": "TFLOP/s", "ms_per_step": round(pms, 4),
            "frac_fp8_peak": round(ptf / FP8_PEAK_TFLOPS, 4),
            "frac_attainable_roofline": round(t_roof / (pms * 1e-3), 4),
            "weight_GBps": round(pbytes / (pms * 1e-3) / 1e9, 1),
            "gate_up_gemm_us": round(pres["gate_up_back_to_back_us"], 2),
            "gate_up_gemm_GBps": round(pres["distinct_mean"] * pw13 /
                                       (pres["gate_up_back_to_back_us"] * 1e-6) / 1e9, 1),
            "per_call_us": {k: round(v, 2) for k, v in pres["per_call_us"].items()},
        }
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
    out["host"] = platform.node()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
