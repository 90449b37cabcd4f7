"""The quantized MoE expert layer -- oracle side (TEST INFRASTRUCTURE ONLY).

Plain NumPy, float64 for every value that is not stored in a narrow format.
The oracle *emulates the quantized pipeline exactly*: it reproduces every
integer and every stored narrow value (expert ids, permutation, INT4 codes and
their fp32 scales, E4M3 codes and their fp32 scales, every bfloat16 rounding
point) and computes every dot product in float64 from those exact values.

Sources (page title, section):
  * "wstewart3/Inkling-Small-W4A8-G128", §1 settings table: symmetric INT4
    weights in groups of 128; dynamic FP8 input activations, one scale per
    token; 256 routed + 2 shared experts; hidden 4096, expert width 2048.
  * same page, §6 "Why this checkpoint also needed recovery": a [2048, 4096]
    projection carries scales [2048, 32], i.e. one scale per (output row,
    128-wide group along the input dimension).
  * same page, §7 "Recover and physically pack INT4": code range [-8, 7] and the
    nibble packing (see ``formats``).
  * same page, intro: INT4 weights with FP8 activations so that the FP8 matrix
    cores stay in use -- the products are FP8 x INT4, accumulated per group.
  * "Inkling-512k-NVFP4-AQLM-hybrid", intro: 256 routed experts per layer, 6
    active; "On-disk tensor format": w13 = fused gate|up, w2 = down.
  * "Inkling 2 Small FP8 for AMD MI300X", "Precision and files": expert weights
    FP8 with one fp32 scale per output channel, scale = max|row| / fmax, and
    dynamic per-token FP8 activations; scale tensor [n_experts, out_channels].
    That card stores E4M3FNUZ with fmax = 240 (MI300X); requant_fnuz_rows
    converts such rows to the OCP E4M3 / 448 rows used here.

Readings where the pages are silent (each listed in the design notes):
  routing is softmax over the k selected logits (softmax-then-top-k with
  renormalization), ties broken toward the lower expert index; the FP8 scale
  divisor is 448 (OCP E4M3 on gfx950); INT4 scale = max|group| / 7 with RNE
  rounding and clamp to [-8, 7]; scales are fp32; the gate/up epilogue is
  h = bf16(silu(g) * u) rounded once; o and y are bf16; the combine is
  y_t = bf16(sum_j w_tj * o_tj + shared_t) summed in slot order.
"""
from __future__ import annotations

import numpy as np

from .formats import (E4M3_MAX, GROUP, bf16_round, e2m1_decode, e4m3_decode, e4m3_encode,
                      e4m3fnuz_decode, fp32, pack_int4, unpack_fp4, unpack_int4)

# ----------------------------------------------------------------- a1: routing


def router_logits(x, w_router):
    """Router scores, the linear layer in front of the top-k selection:
    logits[t, e] = sum_h x[t, h] * Wr[e, h]  ("Inkling-512k-NVFP4-AQLM-hybrid",
    intro: each token is routed to 6 of the 256 experts by its scores).
    x [T, H] and Wr [E, H] hold fp32-representable values; the sum is formed in
    float64 (the kernel accumulates in fp32).  Returns float64 [T, E].
    """
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    w64 = np.asarray(w_router, dtype=np.float32).astype(np.float64)
    return x64 @ w64.T


def route_topk(logits, k: int, bias=None, renormalize: bool = True):
    """Top-k expert selection and routing weights.

    s = logits (+ bias, one fp32 addition); the k largest s per token, ties
    broken toward the lower expert index, listed best first.  Weights:
    renormalize=True  -> w_j = exp(s_j - s_max) / sum over the k selected
    renormalize=False -> w_j = exp(s_j - s_max) / sum over all E experts
    Returns ids int32 [T, k] and weights float64 [T, k].
    """
    s = np.asarray(logits, dtype=np.float32)
    if bias is not None:
        s = (s + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    s = s.astype(np.float64)
    T, E = s.shape
    if not 1 <= k <= E:
        raise ValueError("k out of range")
    # stable sort on -s keeps equal scores in increasing expert order
    order = np.argsort(-s, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(s, ids.astype(np.int64), axis=1)
    smax = s.max(axis=1, keepdims=True)
    num = np.exp(sel - smax)
    den = num.sum(axis=1, keepdims=True) if renormalize else np.exp(s - smax).sum(axis=1, keepdims=True)
    return ids, num / den

# ------------------------------------------------ a2 / a5: per-token FP8 quant


def quant_fp8_per_token(x, block_rows: int = 512):
    """Dynamic per-row FP8 quantization.

    amax_t = max_k |x[t,k]|; s_t = fl32(amax_t / 448); q = E4M3(fl32(x / s_t)).
    Both divisions are IEEE binary32 divisions (the decision that produces an
    integer code is taken in the kernel's precision).  A zero row gets s = 0 and
    all codes 0x00.  x must hold values exactly representable in fp32.
    Returns q uint8 [M, K] and s float32 [M].
    (Rows are processed in blocks only to bound temporary memory.)
    """
    x32 = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x32)):
        raise ValueError("non-finite input")
    M, K = x32.shape
    q = np.zeros((M, K), dtype=np.uint8)
    s = np.zeros(M, dtype=np.float32)
    for r0 in range(0, M, block_rows):
        xb = x32[r0:r0 + block_rows]
        amax = np.abs(xb).max(axis=1)
        sb = (amax / np.float32(E4M3_MAX)).astype(np.float32)
        s[r0:r0 + block_rows] = sb
        nz = np.nonzero(sb > 0)[0]
        if nz.size:
            ratio = (xb[nz] / sb[nz][:, None]).astype(np.float32)
            q[r0 + nz] = e4m3_encode(ratio)
    return q, s


def dequant_fp8_rows(q, s) -> np.ndarray:
    """q * s per row, float64 (used by the brute-force pins)."""
    return e4m3_decode(q) * np.asarray(s, dtype=np.float64)[:, None]

# ------------------------------------------------------ a9: INT4 g128 packing


def _quantize_int4_block(w32, scale_dtype):
    rows, K = w32.shape
    G = K // GROUP
    wg = w32.reshape(rows, G, GROUP)
    a = np.abs(wg).max(axis=2)
    s = (a / np.float32(7.0)).astype(np.float32)
    if scale_dtype == "bf16":
        s = bf16_round(s).astype(np.float32)              # the stored scale, RNE to bfloat16
    c = np.zeros(wg.shape, dtype=np.int8)
    nz = s > 0
    ratio = (wg[nz] / s[nz][:, None]).astype(np.float32)
    c[nz] = np.clip(np.rint(ratio), -8, 7).astype(np.int8)
    return c.reshape(rows, K), s


def quantize_int4_g128(w, block_rows: int = 512, scale_dtype: str = "fp32"):
    """Symmetric INT4 quantization in groups of 128 along the last (input) axis.

    For each row n and group g: a = max|W[n, g]|; s = fl32(a / 7);
    c = clamp(rint(fl32(W / s)), -8, 7) with rint = round half to even;
    a zero group gets s = 0 and codes 0.
    scale_dtype "bf16": the scale is stored as bfloat16, s = bf16(fl32(a / 7))
    (RNE), and the codes are taken against that stored scale -- the 16-bit
    scales that the W4A8 card's payload accounting implies (section 5).
    Returns codes int8 [rows, K] and scales float32 [rows, K/128] (bf16 values
    for "bf16").
    (Rows are processed in blocks only to bound temporary memory.)
    """
    if scale_dtype not in ("fp32", "bf16"):
        raise ValueError(scale_dtype)
    w32 = np.asarray(w, dtype=np.float32)
    rows, K = w32.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    codes = np.empty((rows, K), dtype=np.int8)
    scales = np.empty((rows, K // GROUP), dtype=np.float32)
    for r0 in range(0, rows, block_rows):
        codes[r0:r0 + block_rows], scales[r0:r0 + block_rows] = _quantize_int4_block(
            w32[r0:r0 + block_rows], scale_dtype)
    return codes, scales


def pack_int4_g128(w, scale_dtype: str = "fp32"):
    """quantize_int4_g128 followed by the storage packing: bytes [rows, K/2], scales."""
    codes, s = quantize_int4_g128(w, scale_dtype=scale_dtype)
    return pack_int4(codes), s

# ------------------------------------------------ a8 weights: row-scaled FP8


def quant_fp8_per_row_weights(w):
    """Row-scaled FP8 expert weights: one fp32 scale per output channel.

    Identical arithmetic to the per-token activation quantization applied to
    the rows of W [rows, K]: s_row = fl32(max|row| / 448), wq = E4M3(fl32(W / s)).
    """
    return quant_fp8_per_token(w)



def requant_fnuz_rows(w_fnuz, s_fnuz):
    """Row-scaled E4M3FNUZ weights -> row-scaled OCP E4M3 weights.

    The MI300X card's rows hold E4M3FNUZ codes b with one fp32 scale s per
    output channel (s = max|row| / 240).  Each element's value is formed once in
    fp32, w = fl32(s * fnuz(b)), and the rows of w are quantized exactly as
    quant_fp8_per_row_weights: s' = fl32(max|w| / 448), codes = E4M3(fl32(w / s')).
    The FNUZ NaN code 0x80 is read as 0 (weights hold no NaN).
    Returns codes uint8 [rows, K] and scales float32 [rows].
    """
    b = np.asarray(w_fnuz, dtype=np.uint8)
    s = np.asarray(s_fnuz, dtype=np.float32)
    v = e4m3fnuz_decode(b)
    v = np.where(np.isnan(v), 0.0, v).astype(np.float32)      # exact: 4 significant bits
    w = (s[:, None] * v).astype(np.float32)                   # one fp32 rounding
    return quant_fp8_per_token(w)

# -------------------------------------------------------------- a3: permute


def permute_plan(ids, E: int):
    """Group the (token, slot) rows by expert.

    Row r = t*k + j carries expert ids[t, j].  Rows are ordered by expert, and
    within an expert by increasing r (a stable counting sort).
      counts[e]        rows routed to expert e
      offsets[E+1]     exclusive prefix sum of counts
      sorted_rows[p]   the row r placed at position p
      row_pos[r]       the position p of row r (inverse permutation)
      active           experts with counts > 0, increasing
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_rows = np.argsort(flat, kind="stable").astype(np.int64)
    row_pos = np.empty_like(sorted_rows)
    row_pos[sorted_rows] = np.arange(flat.size)
    active = np.nonzero(counts)[0]
    return {"counts": counts, "offsets": offsets, "sorted_rows": sorted_rows,
            "row_pos": row_pos, "active": active}


def gather_rows(x_q, x_s, sorted_rows, k: int):
    """xp_q[p] = x_q[sorted_rows[p] // k], xp_s likewise."""
    tok = np.asarray(sorted_rows) // k
    return np.asarray(x_q)[tok], np.asarray(x_s)[tok]

# --------------------------------------------------- a4 / a6: grouped GEMMs


def w4a8_rows(a_q, a_s, experts, codes_of, scales_of):
    """W4A8 expert products for a list of rows.

    For row p routed to expert e = experts[p] and output column n:
      P_g  = sum_{k in group g} dec(a_q[p, k]) * c[e, n, k]     (exact in fp64)
      acc  = sum_g s_w[e, n, g] * P_g
      out  = s_a[p] * acc
    codes_of(e) -> int codes [N, K]; scales_of(e) -> fp32 [N, K/128].
    Returns float64 [rows, N].
    """
    a_q = np.asarray(a_q)
    experts = np.asarray(experts)
    a = e4m3_decode(a_q)                                         # [r, K]
    out = None
    for e in np.unique(experts):
        rows = np.nonzero(experts == e)[0]
        c = np.asarray(codes_of(int(e)), dtype=np.float64)       # [N, K]
        s_w = np.asarray(scales_of(int(e)), dtype=np.float64)    # [N, G]
        N, K = c.shape
        G = K // GROUP
        A = a[rows].reshape(len(rows), G, GROUP).transpose(1, 0, 2)   # [G, r, 128]
        C = c.reshape(N, G, GROUP).transpose(1, 2, 0)                 # [G, 128, N]
        partial = np.matmul(A, C)                                     # [G, r, N]
        acc = np.einsum("grn,ng->rn", partial, s_w)
        if out is None:
            out = np.zeros((a_q.shape[0], N), dtype=np.float64)
        out[rows] = np.asarray(a_s, dtype=np.float64)[rows][:, None] * acc
    return out


def fp8row_rows(a_q, a_s, experts, wq_of, srow_of):
    """Row-scaled FP8 expert products for a list of rows.

    out[p, n] = s_a[p] * s_row[e, n] * sum_k dec(a_q[p, k]) * dec(wq[e, n, k]).
    """
    a_q = np.asarray(a_q)
    experts = np.asarray(experts)
    a = e4m3_decode(a_q)
    out = None
    for e in np.unique(experts):
        rows = np.nonzero(experts == e)[0]
        wdec = e4m3_decode(wq_of(int(e)))                         # [N, K]
        srow = np.asarray(srow_of(int(e)), dtype=np.float64)      # [N]
        dot = a[rows] @ wdec.T
        if out is None:
            out = np.zeros((a_q.shape[0], wdec.shape[0]), dtype=np.float64)
        out[rows] = np.asarray(a_s, dtype=np.float64)[rows][:, None] * dot * srow[None, :]
    return out

# ------------------------------------------------------ a4 epilogue: SwiGLU


def nvfp4_dequant(packed, block_scale, scale2):
    """NVFP4 hot-expert weights ("Inkling-512k-NVFP4-AQLM-hybrid", "On-disk tensor
    format" and "Dequant math", hot experts), element by element:

      code(n, k) = (packed[n, k // 2] >> (4 * (k % 2))) & 0xF   (earlier weight in bits 0-3)
      W[n, k]    = e2m1(code(n, k)) * e4m3(block_scale[n, k // 16]) * scale2

    packed [N, K/2] bytes, block_scale [N, K/16] E4M3 bytes, scale2 the expert's
    fp32 scale.  Every factor is exact in float64, and so is the product."""
    packed = np.asarray(packed, dtype=np.uint8)
    N, K = packed.shape[0], 2 * packed.shape[1]
    k = np.arange(K)
    code = (packed[:, k // 2] >> (4 * (k % 2)).astype(np.uint8)) & 0xF      # [N, K]
    bscale = e4m3_decode(np.asarray(block_scale, dtype=np.uint8)[:, k // 16])  # [N, K]
    return e2m1_decode(code) * bscale * float(np.float32(scale2))


def nvfp4_rows(a_q, a_s, experts, packed_of, bscale_of, scale2_of):
    """out[p, n] = a_s[p] * sum_k E4M3(a_q[p, k]) * W_e[n, k] with W_e the NVFP4
    weights of row p's expert (nvfp4_dequant), float64; products exact."""
    a = e4m3_decode(a_q)
    R = a.shape[0]
    out = None
    for e in np.unique(experts):
        rows = np.nonzero(experts == e)[0]
        w = nvfp4_dequant(packed_of(e), bscale_of(e), scale2_of(e))
        blk = (a[rows] @ w.T) * np.asarray(a_s, dtype=np.float64)[rows, None]
        if out is None:
            out = np.zeros((R, w.shape[0]), dtype=np.float64)
        out[rows] = blk
    return out if out is not None else np.zeros((R, 0))


def aqlm_dequant(codes, books, row_scale):
    """AQLM cold-expert weights ("Inkling-512k-NVFP4-AQLM-hybrid", "On-disk tensor
    format" and "Dequant math", cold experts), element by element: input channel k
    of output row n lies in group k // 8 at position k % 8, and

      W[n, k] = row_scale[n] * sum over books b of book_b[codes_b[n, k // 8] & 0xFFFF, k % 8]

    codes: list of [N, K/8] arrays (uint8, or int16 whose negative values stand
    for the unsigned index, hence & 0xFFFF); books: list of fp16 [entries_b, 8];
    row_scale: fp16 [N].  The sum over books and the scaling are exact in float64."""
    N, G = np.asarray(codes[0]).shape
    k = np.arange(8 * G)
    w = np.zeros((N, 8 * G), dtype=np.float64)
    for c, bk in zip(codes, books):
        idx = np.asarray(c).astype(np.int64) & 0xFFFF                      # [N, G]
        book = np.asarray(bk, dtype=np.float16).astype(np.float64)         # [entries, 8]
        w += book[idx[:, k // 8], k % 8]                                   # [N, K]
    return np.asarray(row_scale, dtype=np.float16).astype(np.float64)[:, None] * w


def aqlm_rows(a_q, a_s, experts, codes_of, books, scale_of):
    """out[p, n] = a_s[p] * sum_k E4M3(a_q[p, k]) * W_e[n, k] with W_e the AQLM
    weights of row p's expert (aqlm_dequant; the codebooks are shared by all
    experts of the layer), float64."""
    a = e4m3_decode(a_q)
    R = a.shape[0]
    out = None
    for e in np.unique(experts):
        rows = np.nonzero(experts == e)[0]
        w = aqlm_dequant(codes_of(e), books, scale_of(e))
        blk = (a[rows] @ w.T) * np.asarray(a_s, dtype=np.float64)[rows, None]
        if out is None:
            out = np.zeros((R, w.shape[0]), dtype=np.float64)
        out[rows] = blk
    return out if out is not None else np.zeros((R, 0))


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def silu_mul(o13):
    """h = bf16(silu(g) * u) with g = o13[:, :I] (gate rows first) and u = o13[:, I:].

    One rounding to bfloat16; g and u themselves are not rounded.  Parity unpinned
    beyond tolerance for the GPU side (its exp differs from float64 by ulps).
    """
    o13 = np.asarray(o13, dtype=np.float64)
    I = o13.shape[1] // 2
    return bf16_round(silu(o13[:, :I]) * o13[:, I:])

# ------------------------------------------------------------- a7: combine


def combine(o, row_pos, w, k: int, shared=None):
    """y_t = bf16( sum_{j=0}^{k-1} w[t, j] * o[row_pos[t*k + j]] + shared_t )."""
    o = np.asarray(o, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T = w.shape[0]
    rp = np.asarray(row_pos).reshape(T, k)
    y = np.zeros((T, o.shape[1]), dtype=np.float64)
    for j in range(k):
        y += w[:, j:j + 1] * o[rp[:, j]]
    if shared is not None:
        y += np.asarray(shared, dtype=np.float64)
    return bf16_round(y)

# ------------------------------------------------------ a10: shared experts


def shared_mlp(x, ws13, ws2):
    """bf16 SwiGLU MLP: h = bf16(silu(x Wg^T) * (x Wu^T)); shared = bf16(h Ws2^T).

    ws13 [2S, H] holds the gate rows then the up rows; ws2 [H, S].  All inputs
    are bfloat16 values; products are accumulated in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    o13 = x @ np.asarray(ws13, dtype=np.float64).T
    h = silu_mul(o13)
    return bf16_round(h @ np.asarray(ws2, dtype=np.float64).T)

# ---------------------------------------------------------- the whole layer


def moe_layer(x, logits, k: int, w13=None, w2=None, bias=None, renormalize=True,
              packed13=None, scales13=None, packed2=None, scales2=None,
              fp8row=False, ws13=None, ws2=None, scale_dtype="fp32"):
    """Route -> quantize x -> permute -> gate/up GEMM + SiLU -> quantize h ->
    down GEMM -> combine (+ shared experts).  Returns every intermediate.

    Weights are given either full precision (w13 [E, 2I, H], w2 [E, H, I]) and
    quantized here, or already quantized (packed13/scales13, packed2/scales2).
    With fp8row=True the full-precision weights are quantized row-wise to FP8;
    scale_dtype "bf16" stores the INT4 group scales as bfloat16.
    """
    x = np.asarray(x)
    T, H = x.shape
    E = np.asarray(logits).shape[1]
    res = {}
    ids, w = route_topk(logits, k, bias=bias, renormalize=renormalize)
    res["topk_ids"], res["topk_w"] = ids, w
    xq, xs = quant_fp8_per_token(x)
    res["x_q"], res["x_s"] = xq, xs
    plan = permute_plan(ids, E)
    res.update(plan)
    xp_q, xp_s = gather_rows(xq, xs, plan["sorted_rows"], k)
    res["xp_q"], res["xp_s"] = xp_q, xp_s
    experts = np.repeat(np.arange(E), plan["counts"])

    if fp8row:
        q13, s13, q2, s2 = {}, {}, {}, {}
        for e in plan["active"]:
            q13[e], s13[e] = quant_fp8_per_row_weights(w13[e])
            q2[e], s2[e] = quant_fp8_per_row_weights(w2[e])
        o13 = fp8row_rows(xp_q, xp_s, experts, lambda e: q13[e], lambda e: s13[e])
    else:
        if packed13 is None:
            c13, c2, sc13, sc2 = {}, {}, {}, {}
            for e in plan["active"]:
                c13[e], sc13[e] = quantize_int4_g128(w13[e], scale_dtype=scale_dtype)
                c2[e], sc2[e] = quantize_int4_g128(w2[e], scale_dtype=scale_dtype)
            codes13, codes2 = (lambda e: c13[e]), (lambda e: c2[e])
            sf13, sf2 = (lambda e: sc13[e]), (lambda e: sc2[e])
        else:
            codes13 = lambda e: unpack_int4(packed13[e])  # noqa: E731
            codes2 = lambda e: unpack_int4(packed2[e])  # noqa: E731
            sf13 = lambda e: scales13[e]  # noqa: E731
            sf2 = lambda e: scales2[e]  # noqa: E731
        o13 = w4a8_rows(xp_q, xp_s, experts, codes13, sf13)
    res["o13"] = o13
    h = silu_mul(o13)
    res["h"] = h
    hq, hs = quant_fp8_per_token(h)
    res["h_q"], res["h_s"] = hq, hs
    if fp8row:
        o = fp8row_rows(hq, hs, experts, lambda e: q2[e], lambda e: s2[e])
    else:
        o = w4a8_rows(hq, hs, experts, codes2, sf2)
    o = bf16_round(o)
    res["o"] = o
    shared = None
    if ws13 is not None:
        shared = shared_mlp(x, ws13, ws2)
        res["shared"] = shared
    res["y"] = combine(o, plan["row_pos"], w, k, shared)
    return res


def unquantized_layer(x, logits, k, w13, w2, bias=None, renormalize=True):
    """Sanity reference without any quantization (float64 throughout).  Never gates
    a test; used to log the quantization error."""
    x = np.asarray(x, dtype=np.float64)
    ids, w = route_topk(logits, k, bias=bias, renormalize=renormalize)
    T, H = x.shape
    y = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            o13 = np.asarray(w13[e], dtype=np.float64) @ x[t]
            I = o13.shape[0] // 2
            h = silu(o13[:I]) * o13[I:]
            y[t] += w[t, j] * (np.asarray(w2[e], dtype=np.float64) @ h)
    return y
