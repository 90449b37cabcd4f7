"""Per-call parity of libmoeq against the oracle, on seeded inputs small enough for
the oracle, spanning several tiles with ragged tails and the degenerate cases.

Integer outputs (expert ids, plan, E4M3 codes, INT4 bytes, scales) must be
bit-exact; floating-point outputs must meet rel-L2 <= 2e-3 and
max-abs <= 1e-2 * max|ref|, except where a test states a tighter bound.
"""
import numpy as np
import pytest
import torch

import bit_quantized_moe_top_amd as mq
from oracle import formats as F
from oracle import layer as L
from parity import assert_close, to_np

pytestmark = pytest.mark.gpu


def _dev():
    return torch.device("cuda:0")


# ------------------------------------------------------------- router logits ----
@pytest.mark.parametrize("T,H,E,dtype", [(4, 4096, 256, torch.bfloat16), (16, 4096, 256, torch.float32),
                                         (17, 4096, 256, torch.bfloat16), (130, 528, 100, torch.float32),
                                         (1, 16, 1, torch.float32), (2048, 4096, 256, torch.bfloat16)])
def test_router_logits(T, H, E, dtype):
    g = torch.Generator().manual_seed(T + H + E)
    x = torch.randn(T, H, generator=g).to(dtype)
    w = torch.randn(E, H, generator=g) / 64
    lg = mq.moe_router_logits(x.to(_dev()), w.to(_dev()))
    torch.cuda.synchronize()
    x64, w64 = x.float().numpy(), w.numpy()
    ref = L.router_logits(x64, w64)
    # fp32 accumulation of H products (fused multiply-adds, any order):
    # |err| <= gamma_H * sum_h |x w|, gamma_H = H u / (1 - H u), u = 2^-24
    u = 2.0 ** -24
    bound = (H * u / (1 - H * u)) * (np.abs(x64).astype(np.float64) @ np.abs(w64).astype(np.float64).T)
    err = np.abs(lg.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= bound), float((err / np.maximum(bound, 1e-300)).max())
    # the ids the GPU routes to from its own logits equal the oracle's wherever
    # the oracle's top-(k+1) scores are separated by more than twice the bound
    k = min(6, E)
    ids, _ = mq.moe_route_topk(lg, k)
    torch.cuda.synchronize()
    rid, _ = L.route_topk(ref, k)
    srt = -np.sort(-ref, axis=1)[:, :k + 1]
    gaps = -np.diff(srt, axis=1).min(axis=1) if k < E else np.full(T, np.inf)
    clear = gaps > 2 * bound.max(axis=1)
    assert clear.mean() > 0.9
    np.testing.assert_array_equal(ids.cpu().numpy()[clear], rid[clear])


# ------------------------------------------------------------------ routing ----
@pytest.mark.parametrize("T,E,k", [(37, 256, 6), (16, 8, 2), (5, 1000, 8), (9, 8, 8), (64, 384, 1),
                                   (3, 64, 6)])
@pytest.mark.parametrize("renorm", [True, False])
def test_route_topk(T, E, k, renorm):
    g = torch.Generator().manual_seed(T * 1000 + E + k)
    logits = torch.randn(T, E, generator=g)
    logits[:, 3] = logits[:, 5]                       # ties -> lower index
    if T > 2:
        logits[2, :] = 0.25                           # a fully tied row
    bias = torch.randn(E, generator=g) if E % 2 == 0 else None
    ids, w = mq.moe_route_topk(logits.to(_dev()), k, None if bias is None else bias.to(_dev()), renorm)
    torch.cuda.synchronize()
    rid, rw = L.route_topk(logits.numpy(), k, None if bias is None else bias.numpy(), renorm)
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-6, atol=0)


@pytest.mark.parametrize("E,k", [(256, 6), (1000, 8), (77, 3)])
def test_route_topk_ties_across_lanes_and_signed_zeros(E, k):
    """Equal scores in different lanes and slots go to the lower expert index;
    -0 and +0 are the same score; -inf scores are still selectable."""
    T = 6
    logits = torch.full((T, E), -1.0)
    logits[0, [3, 67, E - 9, E - 1]] = 2.0               # same score, several slots
    logits[1, :] = 0.0
    logits[1, 1::2] = -0.0                              # all zeros of both signs
    logits[2, [E - 1, E - 2, 5]] = torch.tensor([7.0, 7.0, 7.0])
    logits[3, :] = float("-inf")
    logits[3, E // 2] = 0.5                             # one finite score, the rest -inf
    logits[4] = torch.randn(E, generator=torch.Generator().manual_seed(E))
    logits[5, :] = 1e-30
    logits[5, 0] = -1e-30
    ids, w = mq.moe_route_topk(logits.to(_dev()), k)
    torch.cuda.synchronize()
    rid, rw = L.route_topk(logits.numpy(), k, None, True)
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-6, atol=0)


def test_route_empty():
    ids, w = mq.moe_route_topk(torch.zeros(0, 16, device=_dev()), 2)
    assert ids.shape == (0, 2)


# ------------------------------------------------------------ FP8 quantization ----
@pytest.mark.parametrize("M,K,dtype", [(33, 4096, torch.bfloat16), (16, 256, torch.float32),
                                       (7, 2056, torch.bfloat16), (3, 8, torch.float32),
                                       (130, 2048, torch.bfloat16), (5, 8200, torch.bfloat16),
                                       (2, 4104, torch.float32)])
def test_quant_fp8_per_token(M, K, dtype):
    g = torch.Generator().manual_seed(M * 7 + K)
    x = torch.randn(M, K, generator=g) * torch.logspace(-4, 3, M)[:, None]
    x[0] = 0.0                                         # zero row
    if M > 2:
        x[2, :] = -x[2, :].abs()                       # all-negative row
    x = x.to(dtype)
    q, s = mq.quant_fp8_per_token(x.to(_dev()))
    torch.cuda.synchronize()
    rq, rs = L.quant_fp8_per_token(x.to(torch.float32).numpy())
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


def test_e4m3_encoder_boundary_sweep():
    # Rows whose first element is 448 have scale exactly 1, so the codes of the
    # other elements are the encoder applied to the raw values: sweep every
    # midpoint between neighbouring E4M3 values and its fp32 neighbours, every
    # finite bf16 value up to 448, and random fp32 values.
    pos = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    v = [mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
         pos.astype(np.float32)]
    bf = (np.arange(0, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    v.append(bf[bf <= 448])
    v.append(np.random.default_rng(0).uniform(-448, 448, 400_000).astype(np.float32))
    vals = np.concatenate(v + [-x for x in v]).astype(np.float32)
    K = 1024
    n_rows = -(-vals.size // (K - 1))
    x = np.zeros((n_rows, K), np.float32)
    x[:, 0] = 448.0
    flat = x[:, 1:].reshape(-1)
    flat[:vals.size] = vals
    x[:, 1:] = flat.reshape(n_rows, K - 1)
    q, s = mq.quant_fp8_per_token(torch.from_numpy(x).to(_dev()))
    torch.cuda.synchronize()
    assert (s.cpu().numpy() == 1.0).all()
    np.testing.assert_array_equal(q.cpu().numpy()[:, 1:], F.e4m3_encode(x[:, 1:]))


def _rounding_window_rows(n_rows, K, seed):
    """fp32 rows with random non-unit scales whose quotients x / s land within
    +-12 fp32 ulp of every E4M3 rounding midpoint (both signs), so that both the
    reciprocal fast path and the IEEE-division fallback of the encoder, and the
    edge between them (8 ulp), meet values that round differently one ulp apart."""
    rng = np.random.default_rng(seed)
    pos = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)          # 126 midpoints
    offs = np.arange(-12, 13)
    targets = []
    for j in offs:                                               # m + j ulp(m), exact in fp32
        t = mids.copy()
        step = np.float32(np.inf) if j > 0 else np.float32(0)
        for _ in range(abs(int(j))):
            t = np.nextafter(t, step)
        targets.append(t)
    targets = np.concatenate(targets)
    targets = np.concatenate([targets, -targets])
    x = np.zeros((n_rows, K), np.float32)
    amax = np.exp(rng.uniform(np.log(1e-3), np.log(1e3), n_rows)).astype(np.float32)
    # scales below 2^-120 (reciprocal inaccurate: division path), one of them
    # an fp32 subnormal, and a scale of exactly 1/64
    amax[:4] = [1e-35, 2e-34, 2.5e-38, 7.0]
    for r in range(n_rows):
        s = np.float32(amax[r] / np.float32(448.0))
        q = rng.choice(targets, K - 1)
        v = (q * s).astype(np.float32)                           # quotient fl32(v / s) ~ q
        v = np.clip(v, -amax[r], amax[r])                        # the row max stays amax
        x[r, 0] = amax[r] if r % 2 else -amax[r]
        x[r, 1:] = v
    return x


def test_e4m3_encoder_rounding_window_random_scales():
    x = _rounding_window_rows(160, 4096, 5)
    q, s = mq.quant_fp8_per_token(torch.from_numpy(x).to(_dev()))
    torch.cuda.synchronize()
    rq, rs = L.quant_fp8_per_token(x)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    assert (rs != 1.0).all()
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
    # the fused decode front end quantizes x with the same encoder
    T, E, k = 8, 64, 6
    logits = torch.randn(T, E, generator=torch.Generator().manual_seed(3))
    xs = torch.from_numpy(x[:T].copy())
    fused = mq.moe_route_quant_permute(logits.to(_dev()), xs.to(_dev()), k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(fused["x_q"].cpu().numpy(), rq[:T])
    np.testing.assert_array_equal(fused["x_s"].cpu().numpy(), rs[:T])


# ------------------------------------------------- E4M3FNUZ -> OCP requantization ----
@pytest.mark.parametrize("rows,K", [(37, 4096), (50, 2048), (9, 24), (5, 8192), (3, 520),
                                    (4096, 4096)])
def test_requant_fp8_fnuz(rows, K):
    rng = np.random.default_rng(rows * 13 + K)
    b = rng.integers(0, 256, size=(rows, K), dtype=np.uint8)   # includes 0x80 (read as 0)
    b[:, rng.integers(0, K)] = 0x7F                            # a +240 in every row
    s = (rng.random(rows) * 2e-3).astype(np.float32)
    if rows > 3:
        b[1] = 0x00                                            # zero row
        s[2] = 0.0                                             # zero scale
        b[3] = b[3] | 0x80                                     # all-negative row
    w, sc = mq.moe_requant_fp8_fnuz(torch.from_numpy(b).to(_dev()), torch.from_numpy(s).to(_dev()))
    torch.cuda.synchronize()
    rq, rs = L.requant_fnuz_rows(b, s)
    np.testing.assert_array_equal(sc.cpu().numpy(), rs)
    np.testing.assert_array_equal(w.cpu().numpy(), rq)


# -------------------------------------------------------------- INT4 packing ----
@pytest.mark.parametrize("scale_dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("shape", [(3, 256, 384), (1, 16, 128), (5, 128, 4096)])
def test_pack_int4_g128(shape, scale_dtype):
    g = torch.Generator().manual_seed(sum(shape))
    w = torch.randn(*shape, generator=g) * 0.02
    w[0, 1, 128 if shape[2] > 128 else 0:][:128] = 0.0       # a zero group
    w[0, 2, :128] = torch.linspace(-7, 7, 128) * 1e-3          # exact ties at +-0.5 steps
    packed, scales = mq.pack_int4_g128(
        w.to(_dev()), scale_dtype=torch.bfloat16 if scale_dtype == "bf16" else torch.float32)
    torch.cuda.synchronize()
    rows = shape[0] * shape[1]
    rp, rs = L.pack_int4_g128(w.reshape(rows, shape[2]).numpy(), scale_dtype=scale_dtype)
    np.testing.assert_array_equal(scales.cpu().float().numpy().reshape(rows, -1), rs)
    np.testing.assert_array_equal(packed.cpu().numpy().reshape(rows, -1), rp)
    # tiled=True: the same bytes in the GEMMs' tiled order
    tiled, scales_t = mq.pack_int4_g128(
        w.to(_dev()), scale_dtype=torch.bfloat16 if scale_dtype == "bf16" else torch.float32,
        tiled=True)
    torch.cuda.synchronize()
    assert tuple(tiled.shape) == (shape[0], shape[1] // 16, shape[2] // 128, 16, 64)
    np.testing.assert_array_equal(tiled.cpu().numpy(), F.tile_int4(rp.reshape(shape[0], shape[1], -1)))
    np.testing.assert_array_equal(scales_t.cpu().float().numpy().reshape(rows, -1), rs)


@pytest.mark.parametrize("shape", [(1, 16, 128), (3, 48, 384), (2, 4096, 2048), (1, 2048, 4096)])
def test_tile_int4_weights(shape):
    """moe_tile_int4_weights is the oracle's tile_int4 byte for byte, from uint8 rows
    and from the checkpoint's int32 words (the same bytes)."""
    E, N, K = shape
    rng = np.random.default_rng(N + K)
    packed = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    ref = F.tile_int4(packed)
    got = mq.tile_int4_weights(torch.from_numpy(packed).to(_dev()))
    words = torch.from_numpy(packed.view("<i4").copy()).to(_dev())       # int32 [E, N, K/8]
    got_w = mq.tile_int4_weights(words)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), ref)
    np.testing.assert_array_equal(got_w.cpu().numpy(), ref)
    with pytest.raises(ValueError):                     # N not a multiple of 16
        mq.tile_int4_weights(torch.from_numpy(packed[:, :N - 8].copy()).to(_dev()))
    with pytest.raises(ValueError):                     # page-order rows given to a GEMM
        mq.moe_grouped_gemm_w4a8(torch.zeros(1, K, dtype=torch.uint8, device=_dev()),
                                 torch.ones(1, device=_dev()), torch.zeros(64, dtype=torch.int32,
                                                                           device=_dev()),
                                 torch.from_numpy(packed).to(_dev()),
                                 torch.ones(E, N, K // 128, device=_dev()))


# ---------------------------------------------------------------- permute ----
def _check_plan(plan, ids, E, x_q=None, x_s=None, xp_q=None, xp_s=None):
    T, k = ids.shape
    R = T * k
    f = mq.plan_fields(plan.cpu(), E, R)
    ref = L.permute_plan(ids, E)
    hdr = f["header"].numpy()
    assert list(hdr[:7]) == [R, E, len(ref["active"]), int(sum(-(-c // 64) for c in ref["counts"])),
                             T, k, 0]
    np.testing.assert_array_equal(f["offsets"].numpy(), ref["offsets"])
    np.testing.assert_array_equal(f["sorted_rows"].numpy(), ref["sorted_rows"])
    np.testing.assert_array_equal(f["row_pos"].numpy(), ref["row_pos"])
    na = len(ref["active"])
    np.testing.assert_array_equal(f["active"].numpy()[:na], ref["active"])
    tiles = [(e, int(ref["offsets"][e]) + 64 * i) for e in range(E)
             for i in range(-(-int(ref["counts"][e]) // 64))]
    nt = len(tiles)
    np.testing.assert_array_equal(f["tile_expert"].numpy()[:nt], [t[0] for t in tiles])
    np.testing.assert_array_equal(f["tile_row0"].numpy()[:nt], [t[1] for t in tiles])
    if x_q is not None:
        gq, gs = L.gather_rows(x_q, x_s, ref["sorted_rows"], k)
        np.testing.assert_array_equal(xp_q.cpu().numpy(), gq)
        np.testing.assert_array_equal(xp_s.cpu().numpy(), gs)


@pytest.mark.parametrize("T,k,E,mode", [(300, 6, 256, "uniform"), (2048, 6, 256, "uniform"),
                                        (16, 2, 8, "uniform"), (1, 1, 4, "uniform"),
                                        (500, 4, 1000, "uniform"), (200, 3, 16, "hot"),
                                        (4, 6, 256, "uniform"), (1100, 2, 3, "hot")])
def test_permute(T, k, E, mode):
    rng = np.random.default_rng(T + k + E)
    if mode == "hot":                 # most rows on expert 1 -> several tiles for one expert
        ids = np.stack([np.r_[1, rng.choice(np.r_[0, 2:E], k - 1, replace=False)] for _ in range(T)])
    else:
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    ids = ids.astype(np.int32)
    H = 64
    x_q = rng.integers(0, 256, (T, H), dtype=np.uint8)
    x_s = rng.random(T).astype(np.float32)
    plan, xp_q, xp_s = mq.moe_permute(torch.from_numpy(ids).to(_dev()), E,
                                      torch.from_numpy(x_q).to(_dev()),
                                      torch.from_numpy(x_s).to(_dev()))
    torch.cuda.synchronize()
    _check_plan(plan, ids, E, x_q, x_s, xp_q, xp_s)


def test_permute_plan_only_and_empty():
    ids = torch.zeros(0, 6, dtype=torch.int32, device=_dev())
    plan, _, _ = mq.moe_permute(ids, 16)
    torch.cuda.synchronize()
    f = mq.plan_fields(plan.cpu(), 16, 0)
    assert (f["offsets"].numpy() == 0).all() and f["header"][3] == 0


# one-wave plan (R <= 64) with the plan wave outside (T = 4, 5) or inside (T = 8)
# the quantizing waves, workgroup plan (R > 64), a row narrower than a wave
# (H = 48), the largest fused rows (T = 16, H = 2048), the separate-kernel
# fallbacks (T > 16, or rows too long), a single expert, a hot expert, no tokens;
# T > 16 with H % 32 == 0 and H >= 1024 takes the quarter-row quantization and
# scatter: bf16 and fp32 x, one and two chunks per lane (H = 3072: a partial
# second chunk), the plan built in one workgroup (R <= 1024) or placed per row
@pytest.mark.parametrize("T,E,k,H,dtype,hot", [
    (40, 64, 6, 2048, torch.bfloat16, False), (33, 100, 4, 1024, torch.float32, False),
    (200, 256, 6, 4096, torch.float32, True), (1100, 16, 1, 3072, torch.bfloat16, False),
    (4, 256, 6, 4096, torch.bfloat16, False), (1, 8, 2, 256, torch.float32, False),
    (5, 256, 6, 4096, torch.float32, False), (8, 256, 6, 4096, torch.bfloat16, False),
    (16, 1000, 8, 512, torch.bfloat16, False), (8, 64, 8, 48, torch.bfloat16, False),
    (8, 1000, 8, 1024, torch.float32, False), (16, 384, 6, 2048, torch.bfloat16, False),
    (16, 256, 6, 4096, torch.bfloat16, False), (3, 1, 1, 80, torch.bfloat16, False),
    (6, 256, 6, 2048, torch.bfloat16, True), (12, 256, 6, 4096, torch.bfloat16, True),
    (17, 64, 3, 256, torch.bfloat16, False), (300, 256, 6, 128, torch.bfloat16, False),
    (0, 16, 2, 64, torch.float32, False)])
def test_route_quant_permute_fused_matches_separate_and_oracle(T, E, k, H, dtype, hot):
    g = torch.Generator().manual_seed(T * 31 + E + H)
    logits = torch.randn(T, E, generator=g)
    if T > 1:
        logits[1] = logits[0]                       # identical tokens -> equal ids
    bias = torch.randn(E, generator=g) if E % 2 == 0 else None
    if hot:
        bias[5] = 100.0                             # every token routes to expert 5 first
    x = (torch.randn(T, H, generator=g) * 3).to(dtype)
    if T > 2:
        x[2] = 0                                    # zero row
    dl, dx = logits.to(_dev()), x.to(_dev())
    db = None if bias is None else bias.to(_dev())
    fused = mq.moe_route_quant_permute(dl, dx, k, db)
    ids, w = mq.moe_route_topk(dl, k, db)
    xq, xs = mq.quant_fp8_per_token(dx)
    plan, xp_q, xp_s = mq.moe_permute(ids, E, xq, xs)
    torch.cuda.synchronize()
    for name, a, b in (("ids", fused["ids"], ids), ("w", fused["w"], w), ("x_q", fused["x_q"], xq),
                       ("x_s", fused["x_s"], xs), ("xp_q", fused["xp_q"], xp_q),
                       ("xp_s", fused["xp_s"], xp_s)):
        assert torch.equal(a, b), name
    R = T * k
    fp, sp = mq.plan_fields(fused["plan"].cpu(), E, R), mq.plan_fields(plan.cpu(), E, R)
    for name in ("header", "offsets", "sorted_rows", "row_pos"):
        assert torch.equal(fp[name], sp[name]), name
    na = int(fp["header"][2])                       # entries past n_active are unspecified
    assert torch.equal(fp["active"][:na], sp["active"][:na])
    if T:
        rid, rw = L.route_topk(logits.numpy(), k, None if bias is None else bias.numpy())
        np.testing.assert_array_equal(fused["ids"].cpu().numpy(), rid)
        rq, rs = L.quant_fp8_per_token(x.to(torch.float32).numpy())
        np.testing.assert_array_equal(fused["x_q"].cpu().numpy(), rq)
        _check_plan(fused["plan"], rid, E, rq, rs, fused["xp_q"], fused["xp_s"])


# ----------------------------------------------------------- grouped GEMMs ----
def _case_ids(T, k, E, rng, hot=None):
    rows = []
    for _ in range(T):
        if hot is not None:
            rows.append(np.r_[hot, rng.choice([e for e in range(E) if e != hot], k - 1, replace=False)])
        else:
            rows.append(rng.choice(E, k, replace=False))
    return np.stack(rows).astype(np.int32)


def _plan_and_experts(ids, E):
    plan, _, _ = mq.moe_permute(torch.from_numpy(ids).to(_dev()), E)
    ref = L.permute_plan(ids, E)
    experts = np.repeat(np.arange(E), ref["counts"])
    return plan, experts


@pytest.mark.parametrize("T,k,E,N,K,hot", [(40, 2, 8, 256, 256, None),     # R=80 -> 64-row tiles
                                           (4, 6, 16, 256, 512, None),     # R=24 -> decode path
                                           (100, 3, 5, 128, 384, 2),       # expert with >64 rows
                                           (9, 1, 4, 384, 128, None),
                                           # the prefill tile kernels: K = 4096 (gate/up) and
                                           # 2048 (down) with 256-row weight tiles, one expert
                                           # holding 5 row tiles (the last one ragged)
                                           (300, 2, 6, 512, 4096, 1),
                                           (300, 2, 6, 256, 2048, 4)])
def test_w4a8_integer_exact(T, k, E, N, K, hot):
    # unit scales and activations that decode to small integers: every output is
    # an exact integer (|.| < 2^24), so the GPU result must be bit-exact.
    rng = np.random.default_rng(N + K + T)
    ids = _case_ids(T, k, E, rng, hot)
    R = T * k
    plan, experts = _plan_and_experts(ids, E)
    int_code = {v: int(F.e4m3_encode([v])[0]) for v in range(-8, 9)}
    a_int = rng.integers(-8, 9, (R, K))
    a_q = np.vectorize(int_code.get)(a_int).astype(np.uint8)
    codes = rng.integers(-8, 8, (E, N, K)).astype(np.int8)      # includes -8 (GPTQ range)
    packed = F.pack_int4(codes)
    ones_w = np.ones((E, N, K // 128), np.float32)
    for epi in (mq.EPI_NONE, mq.EPI_SILU_MUL):
        out = mq.moe_grouped_gemm_w4a8(
            torch.from_numpy(a_q).to(_dev()), torch.ones(R, device=_dev()), plan,
            mq.tile_int4_weights(torch.from_numpy(packed).to(_dev())),
            torch.from_numpy(ones_w).to(_dev()),
            epilogue=epi, out_dtype=torch.float32 if epi == mq.EPI_NONE else torch.bfloat16)
        torch.cuda.synchronize()
        ref = L.w4a8_rows(a_q, np.ones(R, np.float32), experts, lambda e: codes[e],
                          lambda e: ones_w[e])
        if epi == mq.EPI_NONE:
            np.testing.assert_array_equal(out.cpu().numpy(), ref)
        else:
            assert_close(to_np(out), L.silu_mul(ref), rel=4e-3, max_abs_frac=1e-2, what="silu")


@pytest.mark.parametrize("fmt", ["w4a8", "fp8row", "w4a8_bf16s"])
@pytest.mark.parametrize("T,k,E,N,K,hot", [(40, 2, 8, 256, 256, None), (4, 6, 16, 256, 512, None),
                                           (100, 3, 5, 256, 384, 2), (50, 6, 64, 128, 256, None),
                                           (70, 2, 4, 384, 4096, 1), (100, 3, 6, 512, 2048, 2),
                                           (4, 6, 24, 512, 4096, None),
                                           # prefill tile kernels (R > 192): K = 4096 and 2048,
                                           # N a multiple of 256, an expert with 5 row tiles
                                           (300, 2, 6, 512, 4096, 1), (260, 3, 7, 256, 2048, 3),
                                           # 128-row weight tiles (N % 256 != 0), looped K sweep,
                                           # 40 experts split over the 8 per-XCD runs
                                           (400, 4, 40, 384, 1024, 5)])
def test_grouped_gemm_random(fmt, T, k, E, N, K, hot):
    rng = np.random.default_rng(E + N + K + T)
    ids = _case_ids(T, k, E, rng, hot)
    R = T * k
    plan, experts = _plan_and_experts(ids, E)
    x = (rng.standard_normal((R, K)) * rng.uniform(0.1, 10, (R, 1))).astype(np.float32)
    a_q, a_s = L.quant_fp8_per_token(x)
    w = (rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    ws_t = lambda a: torch.from_numpy(a).to(_dev())  # noqa
    if fmt in ("w4a8", "w4a8_bf16s"):
        sdt = "bf16" if fmt == "w4a8_bf16s" else "fp32"
        cs = [L.quantize_int4_g128(w[e], scale_dtype=sdt) for e in range(E)]
        wq = np.stack([F.pack_int4(c) for c, _ in cs])
        ws = np.stack([s for _, s in cs])
        if sdt == "bf16":                       # the scales are bf16 values: exact conversion
            ws_t = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(_dev())  # noqa
        fn = mq.moe_grouped_gemm_w4a8
        ref_fn = lambda: L.w4a8_rows(a_q, a_s, experts, lambda e: cs[e][0], lambda e: cs[e][1])  # noqa
    else:
        qs = [L.quant_fp8_per_row_weights(w[e]) for e in range(E)]
        wq = np.stack([q for q, _ in qs])
        ws = np.stack([s for _, s in qs])
        fn = mq.moe_grouped_gemm_fp8row
        ref_fn = lambda: L.fp8row_rows(a_q, a_s, experts, lambda e: qs[e][0], lambda e: qs[e][1])  # noqa
    ref = ref_fn()
    dq = lambda a: torch.from_numpy(a).to(_dev())  # noqa
    wt = dq(wq) if fmt == "fp8row" else mq.tile_int4_weights(dq(wq))
    out32 = fn(dq(a_q), dq(a_s), plan, wt, ws_t(ws), epilogue=mq.EPI_NONE,
               out_dtype=torch.float32)
    outbf = fn(dq(a_q), dq(a_s), plan, wt, ws_t(ws), epilogue=mq.EPI_NONE,
               out_dtype=torch.bfloat16)
    h = fn(dq(a_q), dq(a_s), plan, wt, ws_t(ws), epilogue=mq.EPI_SILU_MUL)
    torch.cuda.synchronize()
    assert_close(to_np(out32), ref, rel=1e-4, max_abs_frac=1e-4, what="fp32 out")
    assert_close(to_np(outbf), F.bf16_round(ref), what="bf16 out")
    assert_close(to_np(h), L.silu_mul(ref), what="silu_mul")
    # determinism: a second run is bitwise identical
    h2 = fn(dq(a_q), dq(a_s), plan, wt, ws_t(ws), epilogue=mq.EPI_SILU_MUL)
    assert torch.equal(h, h2)


# ------------------------------------------------------------- NVFP4 experts ----
def _nvfp4_case(T, k, E, N, K, hot, seed, pow2_scales=False):
    rng = np.random.default_rng(seed)
    ids = _case_ids(T, k, E, rng, hot)
    plan, experts = _plan_and_experts(ids, E)
    codes = rng.integers(0, 16, (E, N, K)).astype(np.uint8)
    if pow2_scales:                                   # 2^-3 .. 2^2 (E4M3 0x20 .. 0x48, m = 0)
        bs = (rng.integers(4, 10, (E, N, K // 16)) * 8).astype(np.uint8)
        s2 = np.ones(E, np.float32)
    else:
        bs = rng.integers(0x20, 0x50, (E, N, K // 16)).astype(np.uint8)
        s2 = (rng.random(E) * 0.02 + 1e-3).astype(np.float32)
    return rng, plan, experts, codes, F.pack_fp4(codes), bs, s2


@pytest.mark.parametrize("T,k,E,N,K,hot", [(4, 6, 16, 256, 512, None), (40, 2, 8, 384, 256, 1),
                                           (100, 3, 6, 512, 2048, 2), (4, 6, 8, 128, 6144, None)])
def test_nvfp4_gemm_random(T, k, E, N, K, hot):
    rng, plan, experts, codes, packed, bs, s2 = _nvfp4_case(T, k, E, N, K, hot, N + K + T)
    R = T * k
    x = (rng.standard_normal((R, K)) * rng.uniform(0.1, 10, (R, 1))).astype(np.float32)
    a_q, a_s = L.quant_fp8_per_token(x)
    ref = L.nvfp4_rows(a_q, a_s, experts, lambda e: packed[e], lambda e: bs[e], lambda e: s2[e])
    d = lambda a: torch.from_numpy(a).to(_dev())  # noqa
    args = (d(a_q), d(a_s), plan, d(packed), d(bs), d(s2))
    out32 = mq.moe_grouped_gemm_nvfp4(*args, epilogue=mq.EPI_NONE, out_dtype=torch.float32)
    outbf = mq.moe_grouped_gemm_nvfp4(*args, epilogue=mq.EPI_NONE)
    h = mq.moe_grouped_gemm_nvfp4(*args, epilogue=mq.EPI_SILU_MUL)
    torch.cuda.synchronize()
    assert_close(to_np(out32), ref, rel=1e-4, max_abs_frac=1e-4, what="fp32 out")
    assert_close(to_np(outbf), F.bf16_round(ref), what="bf16 out")
    assert_close(to_np(h), L.silu_mul(ref), what="silu_mul")
    h2 = mq.moe_grouped_gemm_nvfp4(*args, epilogue=mq.EPI_SILU_MUL)
    assert torch.equal(h, h2)


@pytest.mark.parametrize("T,k,E,N,K,hot", [(8, 2, 4, 128, 1024, None), (70, 1, 2, 256, 512, 0)])
def test_nvfp4_gemm_exact(T, k, E, N, K, hot):
    # small-integer activations, power-of-two block scales, scale2 = 1, unit
    # activation scales: every product and partial sum is a multiple of 2^-4
    # below 2^20, so the fp32 result is exact and must equal the oracle bit for bit
    rng, plan, experts, codes, packed, bs, s2 = _nvfp4_case(T, k, E, N, K, hot, K + T, True)
    R = T * k
    int_code = {v: int(F.e4m3_encode([v])[0]) for v in range(-8, 9)}
    a_q = np.vectorize(int_code.get)(rng.integers(-8, 9, (R, K))).astype(np.uint8)
    a_s = np.ones(R, np.float32)
    ref = L.nvfp4_rows(a_q, a_s, experts, lambda e: packed[e], lambda e: bs[e], lambda e: s2[e])
    d = lambda a: torch.from_numpy(a).to(_dev())  # noqa
    out = mq.moe_grouped_gemm_nvfp4(d(a_q), d(a_s), plan, d(packed), d(bs), d(s2),
                                    epilogue=mq.EPI_NONE, out_dtype=torch.float32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), ref)


# -------------------------------------------------------------- AQLM experts ----
def _aqlm_case(E, N, K, books, rng, int_books=False):
    codes, cbs = [], []
    for entries in books:
        if int_books:
            bk = rng.integers(-4, 5, (entries, 8)).astype(np.float16)
        else:
            bk = (rng.standard_normal((entries, 8)) * 0.05).astype(np.float16)
        if entries > 256:
            c = rng.integers(0, entries, (E, N, K // 8)).astype(np.int64)
            c = np.where(c >= 32768, c - 65536, c).astype(np.int16)     # int16 wrap
        else:
            c = rng.integers(0, entries, (E, N, K // 8)).astype(np.uint8)
        codes.append(c)
        cbs.append(bk)
    return codes, cbs


@pytest.mark.parametrize("books", [(65536,), (65536, 256), (200,), (300, 70)])
@pytest.mark.parametrize("T,k,E,N,K,hot", [(4, 6, 16, 256, 512, None), (40, 2, 6, 384, 1024, 1)])
def test_aqlm_gemm_random(books, T, k, E, N, K, hot):
    rng = np.random.default_rng(N + K + T + sum(books))
    ids = _case_ids(T, k, E, rng, hot)
    plan, experts = _plan_and_experts(ids, E)
    R = T * k
    codes, cbs = _aqlm_case(E, N, K, books, rng)
    sc = (rng.random((E, N)) + 0.5).astype(np.float16)
    x = (rng.standard_normal((R, K)) * rng.uniform(0.1, 10, (R, 1))).astype(np.float32)
    a_q, a_s = L.quant_fp8_per_token(x)
    ref = L.aqlm_rows(a_q, a_s, experts, lambda e: [c[e] for c in codes], cbs, lambda e: sc[e])
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(_dev())  # noqa
    args = (d(a_q), d(a_s), plan, [d(c) for c in codes], [d(b) for b in cbs], d(sc))
    out32 = mq.moe_grouped_gemm_aqlm(*args, epilogue=mq.EPI_NONE, out_dtype=torch.float32)
    h = mq.moe_grouped_gemm_aqlm(*args, epilogue=mq.EPI_SILU_MUL)
    torch.cuda.synchronize()
    assert_close(to_np(out32), ref, rel=1e-4, max_abs_frac=1e-4, what="fp32 out")
    assert_close(to_np(h), L.silu_mul(ref), what="silu_mul")


def test_aqlm_gemm_exact():
    # integer codebook entries, small-integer activations, unit scales: exact sums
    rng = np.random.default_rng(77)
    T, k, E, N, K = 8, 2, 4, 128, 512
    ids = _case_ids(T, k, E, rng)
    plan, experts = _plan_and_experts(ids, E)
    R = T * k
    codes, cbs = _aqlm_case(E, N, K, (65536, 256), rng, int_books=True)
    sc = np.ones((E, N), np.float16)
    int_code = {v: int(F.e4m3_encode([v])[0]) for v in range(-8, 9)}
    a_q = np.vectorize(int_code.get)(rng.integers(-8, 9, (R, K))).astype(np.uint8)
    a_s = np.ones(R, np.float32)
    ref = L.aqlm_rows(a_q, a_s, experts, lambda e: [c[e] for c in codes], cbs, lambda e: sc[e])
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(_dev())  # noqa
    out = mq.moe_grouped_gemm_aqlm(d(a_q), d(a_s), plan, [d(c) for c in codes],
                                   [d(b) for b in cbs], d(sc), epilogue=mq.EPI_NONE,
                                   out_dtype=torch.float32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), ref)


def test_hybrid_nvfp4_and_aqlm_slabs():
    # hot experts as NVFP4 slabs, cold ones as AQLM slabs (the hybrid card's
    # hot_ids / cold_ids); each call fills only the rows of its own experts
    rng = np.random.default_rng(5)
    T, k, E, N, K = 12, 4, 10, 256, 512
    ids = _case_ids(T, k, E, rng)
    plan, experts = _plan_and_experts(ids, E)
    R = T * k
    hot_ids = np.array([1, 4, 7], np.int32)
    cold_ids = np.array([e for e in range(E) if e not in hot_ids], np.int32)
    hot_of = np.full(E, -1, np.int32); hot_of[hot_ids] = np.arange(len(hot_ids))
    cold_of = np.full(E, -1, np.int32); cold_of[cold_ids] = np.arange(len(cold_ids))
    packed = F.pack_fp4(rng.integers(0, 16, (len(hot_ids), N, K)).astype(np.uint8))
    bs = rng.integers(0x20, 0x50, (len(hot_ids), N, K // 16)).astype(np.uint8)
    s2 = (rng.random(len(hot_ids)) * 0.02 + 1e-3).astype(np.float32)
    codes, cbs = _aqlm_case(len(cold_ids), N, K, (65536, 256), rng)
    sc = (rng.random((len(cold_ids), N)) + 0.5).astype(np.float16)
    x = rng.standard_normal((R, K)).astype(np.float32)
    a_q, a_s = L.quant_fp8_per_token(x)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(_dev())  # noqa
    out = torch.full((R, N), float("nan"), device=_dev())
    mq.moe_grouped_gemm_nvfp4(d(a_q), d(a_s), plan, d(packed), d(bs), d(s2), epilogue=mq.EPI_NONE,
                              out_dtype=torch.float32, out=out, slab_of=d(hot_of))
    mq.moe_grouped_gemm_aqlm(d(a_q), d(a_s), plan, [d(c) for c in codes], [d(b) for b in cbs],
                             d(sc), epilogue=mq.EPI_NONE, out_dtype=torch.float32, out=out,
                             slab_of=d(cold_of))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert not np.isnan(got).any()                    # every row written by exactly one format
    hot_rows = np.isin(experts, hot_ids)
    ref_h = L.nvfp4_rows(a_q[hot_rows], a_s[hot_rows], experts[hot_rows],
                         lambda e: packed[hot_of[e]], lambda e: bs[hot_of[e]],
                         lambda e: s2[hot_of[e]])
    ref_c = L.aqlm_rows(a_q[~hot_rows], a_s[~hot_rows], experts[~hot_rows],
                        lambda e: [c[cold_of[e]] for c in codes], cbs, lambda e: sc[cold_of[e]])
    assert_close(got[hot_rows], ref_h, rel=1e-4, max_abs_frac=1e-4, what="hot rows")
    assert_close(got[~hot_rows], ref_c, rel=1e-4, max_abs_frac=1e-4, what="cold rows")


# ------------------------------------------------------------------ combine ----
def _assert_combine_close(got, ref, o, row_pos, w, k, shared):
    """The GPU sums in fp32 (slot order) and rounds once to bf16; the reference
    rounds the exact sum.  Bound: one bf16 ulp of the result, plus the fp32
    accumulation error of <= k + 1 terms (k u sum|terms|, u = 2^-24), which
    matters only where the terms cancel."""
    T = w.shape[0]
    rp = np.asarray(row_pos).reshape(T, k)
    mag = np.zeros_like(ref, dtype=np.float64)
    for j in range(k):
        mag += np.abs(w[:, j:j + 1].astype(np.float64) * np.asarray(o, dtype=np.float64)[rp[:, j]])
    if shared is not None:
        mag += np.abs(np.asarray(shared, dtype=np.float64))
    bound = np.abs(ref) * 2.0 ** -7 + (k + 1) * 2.0 ** -24 * mag * 2.0 + 1e-30
    assert np.all(np.abs(got - ref) <= bound)
    assert np.mean(got == ref) > 0.99


# k = MOEQ_MAX_TOPK, and a row narrower than one block of 256 threads x 8 columns
@pytest.mark.parametrize("T,k,E,H,shared", [(33, 6, 256, 4096, False), (16, 2, 8, 256, True),
                                            (5, 1, 3, 8, False), (7, 8, 16, 2056, True)])
def test_combine(T, k, E, H, shared):
    rng = np.random.default_rng(T + H)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    plan, _, _ = mq.moe_permute(torch.from_numpy(ids).to(_dev()), E)
    ref_plan = L.permute_plan(ids, E)
    o = F.bf16_round(rng.standard_normal((T * k, H)))
    w = rng.random((T, k)).astype(np.float32)
    sh = F.bf16_round(rng.standard_normal((T, H))) if shared else None
    y = mq.moe_combine(torch.from_numpy(o).to(torch.bfloat16).to(_dev()), plan,
                       torch.from_numpy(w).to(_dev()),
                       None if sh is None else torch.from_numpy(sh).to(torch.bfloat16).to(_dev()))
    torch.cuda.synchronize()
    ref = L.combine(o, ref_plan["row_pos"], w, k, sh)
    _assert_combine_close(to_np(y), ref, o, ref_plan["row_pos"], w, k, sh)


@pytest.mark.parametrize("T,k,E,H", [(7, 8, 16, 2056), (3, 2, 4, 64), (40, 6, 256, 512)])
def test_permute_and_combine_drop_out_of_range_ids(T, k, E, H):
    """Ids outside [0, E) (never produced by routing) are dropped: the other rows
    keep their stable expert order, the dropped ones get row_pos -1, are counted
    in the plan header, and add nothing in the combine.  Expected values: the
    oracle's plan with every such id moved to an extra expert E sorted last."""
    rng = np.random.default_rng(T * k + E)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[0, k - 1] = -1
    ids[T - 1, 0] = E
    ids[T // 2, k // 2] = E + 7
    R = T * k
    valid = (ids >= 0) & (ids < E)
    n_valid = int(valid.sum())
    plan, _, _ = mq.moe_permute(torch.from_numpy(ids).to(_dev()), E)
    torch.cuda.synchronize()
    ref = L.permute_plan(np.where(valid, ids, E), E + 1)
    pf = {name: to_np(v) for name, v in mq.plan_fields(plan, E, R).items()}
    assert int(pf["header"][6]) == R - n_valid                  # dropped rows
    np.testing.assert_array_equal(pf["offsets"], ref["offsets"][:E + 1])
    flat_valid = valid.reshape(-1)
    np.testing.assert_array_equal(pf["row_pos"][flat_valid], ref["row_pos"][flat_valid])
    assert np.all(pf["row_pos"][~flat_valid] == -1)
    np.testing.assert_array_equal(pf["sorted_rows"][:n_valid], ref["sorted_rows"][:n_valid])
    np.testing.assert_array_equal(pf["active"][:len(ref["active"]) - 1], ref["active"][:-1])

    o = F.bf16_round(rng.standard_normal((R, H)))
    w = rng.random((T, k)).astype(np.float32)
    sh = F.bf16_round(rng.standard_normal((T, H)))
    y = mq.moe_combine(torch.from_numpy(o).to(torch.bfloat16).to(_dev()), plan,
                       torch.from_numpy(w).to(_dev()),
                       torch.from_numpy(sh).to(torch.bfloat16).to(_dev()))
    torch.cuda.synchronize()
    # a dropped slot adds an exact zero: its weight is 0, its row any valid one
    rp = np.where(flat_valid, ref["row_pos"], 0)
    w0 = np.where(valid, w, 0.0)
    y_ref = L.combine(o, rp, w0, k, sh)
    _assert_combine_close(to_np(y), y_ref, o, rp, w0, k, sh)


# ------------------------------------------------------------- shared GEMM ----
# With K % 64 == 0 and at least 256 tiles of 256 rows: 256x256 tiles (ring of 2
# slots of 64 K), else 256x128 (ring of 3); ragged last row tile, one slot,
# fewer slots than the ring holds and more.  Otherwise M < 256 takes the
# 128x128 small-tile kernel and larger M the 128-row kernel: 128x256 tiles when
# they make >= 512 workgroups, else 128x128 (ragged last row tile, one K step,
# several column tiles)
@pytest.mark.parametrize("M,N,K", [(37, 256, 256), (128, 512, 4096), (200, 128, 96),
                                   (256, 256, 64), (300, 512, 320), (777, 1024, 192),
                                   (513, 768, 4096), (256, 128, 32), (2000, 8192, 96),
                                   (2000, 8192, 128), (1000, 8192, 192), (256, 32768, 64),
                                   (300, 16384, 192), (512, 32768, 64), (2000, 8192, 320),
                                   (1000, 8192, 448)])
def test_shared_gemm_bf16(M, N, K):
    g = torch.Generator().manual_seed(M + N + K)
    a = torch.randn(M, K, generator=g).to(torch.bfloat16)
    w = (torch.randn(N, K, generator=g) * 0.05).to(torch.bfloat16)
    none = mq.moe_shared_gemm_bf16(a.to(_dev()), w.to(_dev()), mq.EPI_NONE)
    silu = mq.moe_shared_gemm_bf16(a.to(_dev()), w.to(_dev()), mq.EPI_SILU_MUL)
    torch.cuda.synchronize()
    acc = a.double().numpy() @ w.double().numpy().T
    assert_close(to_np(none), F.bf16_round(acc), what="none")
    assert_close(to_np(silu), L.silu_mul(acc), what="silu")


@pytest.mark.parametrize("T,H,S", [(64, 256, 128), (300, 512, 384), (1024, 1024, 512)])
def test_shared_mlp_kernels_vs_oracle(T, H, S):
    """The shared experts as the layer runs them -- moe_shared_gemm_bf16 with the
    SiLU-gated epilogue on ws13 [2S, H], then plain on ws2 [H, S] -- against the
    oracle's shared_mlp (h rounded to bf16 once, fp64 products).  Covers the
    small-tile (M < 256) and large-tile kernels and a ragged last row tile."""
    g = torch.Generator().manual_seed(T + H + S)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    ws13 = (torch.randn(2 * S, H, generator=g) * 0.05).to(torch.bfloat16)
    ws2 = (torch.randn(H, S, generator=g) * 0.05).to(torch.bfloat16)
    h = mq.moe_shared_gemm_bf16(x.to(_dev()), ws13.to(_dev()), mq.EPI_SILU_MUL)
    out = mq.moe_shared_gemm_bf16(h, ws2.to(_dev()), mq.EPI_NONE)
    torch.cuda.synchronize()
    ref = L.shared_mlp(x.float().numpy(), ws13.float().numpy(), ws2.float().numpy())
    assert_close(to_np(out), ref, what="shared")


# ------------------------------------------------------- read-bandwidth probe ----
@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 3 << 20, (64 << 20) + 16])
def test_read_bandwidth_probe_reads_every_word(nbytes):
    """The probe's sink words XOR to the XOR of every 32-bit word of the buffer
    (so it really reads all of it, ragged tails included)."""
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32).copy()).to(_dev())
    sink = mq.moe_read_bandwidth_probe(buf)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(words))

