"""The oracle over a whole full-size layer, every routed row, for the parity tests.

A routed row's h, h codes and o depend only on the row's own activations and
its expert's weights, so the oracle's per-expert functions (w4a8_rows /
fp8row_rows, silu_mul, quant_fp8_per_token, bf16 rounding) are evaluated for
one expert at a time, experts in parallel threads; the results are assembled in
plan order and combined with the oracle's combine.  This is the same sequence
as oracle.layer.moe_layer, spread over experts: no value is computed
differently, only in another thread.  The fp32 expert weights are regenerated
by the workload generator on the device that generated the GPU path's weights
(the same tensors), one expert at a time.

Test infrastructure only (imports the oracle); never used by the product path.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import time

import numpy as np
import torch
from threadpoolctl import threadpool_limits

import workloads as W
from oracle import formats as F
from oracle import layer as L


def host_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _expert_rows(e, rows, xp_q, xp_s, w13, w2, fmt, other_codes=None):
    """h, h_q, h_s, o of the rows routed to expert e (oracle functions only), and,
    given another quantization of those rows' h (codes, scales), the bound
    o_bound on how far the down projection of it may lie from the oracle's o."""
    experts = np.full(len(rows), e)
    if fmt == "fp8row":
        q13, s13 = L.quant_fp8_per_row_weights(w13)
        q2, s2 = L.quant_fp8_per_row_weights(w2)
        o13 = L.fp8row_rows(xp_q[rows], xp_s[rows], experts, lambda _: q13, lambda _: s13)
    else:
        sdt = "bf16" if fmt == "w4a8_bf16s" else "fp32"
        c13, s13 = L.quantize_int4_g128(w13, scale_dtype=sdt)
        c2, s2 = L.quantize_int4_g128(w2, scale_dtype=sdt)
        o13 = L.w4a8_rows(xp_q[rows], xp_s[rows], experts, lambda _: c13, lambda _: s13)
    h = L.silu_mul(o13)
    hq, hs = L.quant_fp8_per_token(h)
    if fmt == "fp8row":
        o = L.fp8row_rows(hq, hs, experts, lambda _: q2, lambda _: s2)
    else:
        o = L.w4a8_rows(hq, hs, experts, lambda _: c2, lambda _: s2)
    o_bound = None
    if other_codes is not None:
        if fmt == "fp8row":
            wdeq = np.abs(L.dequant_fp8_rows(q2, s2))                        # [H, I]
        else:
            wdeq = np.abs(c2.astype(np.float64) *
                          np.repeat(s2.astype(np.float64), 128, axis=1))
        a_ref = L.dequant_fp8_rows(hq, hs)                                    # [rows, I]
        a_oth = L.dequant_fp8_rows(*other_codes)
        # the activations' difference carried through |W|, plus an fp32
        # accumulation allowance of 2^-12 of the absolute sums
        o_bound = np.abs(a_oth - a_ref) @ wdeq.T * (1 + 2.0 ** -10) + \
            2.0 ** -12 * ((np.abs(a_oth) + np.abs(a_ref)) @ wdeq.T)
    return h, hq, hs, F.bf16_round(o), o_bound


def full_layer(cfg, x, logits, bias, device, ws13=None, ws2=None, log=print, other_h=None):
    """Every intermediate of the layer for all T tokens: dict with topk_ids, topk_w,
    x_q, x_s, the plan arrays, h, h_q, h_s, o, (shared), y.

    other_h: (h codes [R, I], h scales [R]) of another correct evaluation of the
    layer (the GPU's), whose h may round differently from the oracle's where h
    lands within an ulp of a rounding point.  They do not enter any oracle
    value; they only set the tolerance o_bound [R, H]: |W2| times the difference
    of the two dequantized activation rows, plus an fp32 accumulation allowance
    (zero difference where the two quantizations of a row agree)."""
    t0 = time.time()
    res = {}
    ids, w = L.route_topk(logits, cfg.k, bias)
    res["topk_ids"], res["topk_w"] = ids, w
    xq, xs = L.quant_fp8_per_token(x)
    res["x_q"], res["x_s"] = xq, xs
    plan = L.permute_plan(ids, cfg.E)
    res.update(plan)
    xp_q, xp_s = L.gather_rows(xq, xs, plan["sorted_rows"], cfg.k)
    R = cfg.R
    h = np.zeros((R, cfg.I))
    hq = np.zeros((R, cfg.I), np.uint8)
    hs = np.zeros(R, np.float32)
    o = np.zeros((R, cfg.H))
    o_bound = np.zeros((R, cfg.H)) if other_h is not None else None
    active = [int(e) for e in plan["active"]]
    nthr = host_threads()
    chunk = 2 * nthr
    with threadpool_limits(1), cf.ThreadPoolExecutor(nthr) as pool:
        for c0 in range(0, len(active), chunk):
            jobs = []
            for e in active[c0:c0 + chunk]:
                rows = np.arange(plan["offsets"][e], plan["offsets"][e + 1])
                w13 = W.expert_weight(cfg, "w13", e, device).cpu().numpy()
                w2 = W.expert_weight(cfg, "w2", e, device).cpu().numpy()
                oth = None if other_h is None else (other_h[0][rows], other_h[1][rows])
                jobs.append((rows, pool.submit(_expert_rows, e, rows, xp_q, xp_s, w13, w2,
                                               cfg.weight_format, oth)))
            for rows, fut in jobs:
                h[rows], hq[rows], hs[rows], o[rows], ob = fut.result()
                if ob is not None:
                    o_bound[rows] = ob
    res["h"], res["h_q"], res["h_s"], res["o"] = h, hq, hs, o
    if o_bound is not None:
        res["o_bound"] = o_bound
    shared = None
    if ws13 is not None:
        shared = L.shared_mlp(x, ws13, ws2)
        res["shared"] = shared
    res["y"] = L.combine(o, plan["row_pos"], w, cfg.k, shared)
    log(f"[{cfg.name}] oracle over {len(active)} experts, {R} rows: {time.time() - t0:.1f} s "
        f"on {nthr} host threads")
    return res
