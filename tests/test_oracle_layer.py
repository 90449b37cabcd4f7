"""Pins for oracle/layer.py.

Each pin checks the oracle against something other than itself: pure-Python
brute force on tiny inputs, closed forms and invariants of the stated formulas,
special cases with exactly known answers, library routines (scipy, torch), an
algebraically different evaluation order (dequantize-then-matmul), and the
shape facts printed on the Inkling-Small W4A8 card.
"""
import os

import numpy as np
import pytest
import scipy.special
import torch

import workloads as W
from oracle import formats as F
from oracle import layer as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_shapes():
    d = {}
    with open(os.path.join(GOLDEN, "inkling_small_shapes.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                d[k] = float(v)
    return d


# --------------------------------------------------------------- routing ----
def _route_brute(s_row, k):
    order = sorted(range(len(s_row)), key=lambda e: (-float(s_row[e]), e))
    return order[:k]


def test_router_logits_brute_force_and_integer_case():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((3, 5)).astype(np.float32)
    w = rng.standard_normal((4, 5)).astype(np.float32)
    got = L.router_logits(x, w)
    for t in range(3):
        for e in range(4):
            want = sum(float(x[t, h]) * float(w[e, h]) for h in range(5))
            assert abs(got[t, e] - want) <= 1e-15 * sum(abs(float(x[t, h]) * float(w[e, h]))
                                                          for h in range(5))
    xi = rng.integers(-9, 10, (6, 128)).astype(np.float32)          # exact in any order
    wi = rng.integers(-9, 10, (7, 128)).astype(np.float32)
    gi = L.router_logits(xi, wi)
    want = [[sum(int(a) * int(b) for a, b in zip(xi[t], wi[e])) for e in range(7)] for t in range(6)]
    assert np.array_equal(gi, np.array(want, dtype=np.float64))


def test_route_matches_brute_force_sort():
    rng = np.random.default_rng(3)
    for T, E, k in [(7, 8, 2), (5, 16, 6), (4, 256, 6), (3, 5, 5)]:
        logits = rng.standard_normal((T, E)).astype(np.float32)
        logits[:, 1] = logits[:, 2]          # plant ties
        bias = rng.standard_normal(E).astype(np.float32)
        for b in (None, bias):
            ids, w = L.route_topk(logits, k, bias=b)
            s = logits if b is None else (logits + b).astype(np.float32)
            for t in range(T):
                assert list(ids[t]) == _route_brute(s[t], k)
                ex = [np.exp(float(s[t, e]) - float(s[t].max())) for e in ids[t]]
                np.testing.assert_allclose(w[t], np.array(ex) / sum(ex), rtol=1e-14)


def test_route_ties_go_to_lower_index_and_weights_sum_to_one():
    logits = np.zeros((3, 10), dtype=np.float32)
    ids, w = L.route_topk(logits, 4)
    assert (ids == np.arange(4)).all()
    np.testing.assert_allclose(w, 0.25)
    ids, w = L.route_topk(np.random.default_rng(0).standard_normal((9, 12)), 1)
    np.testing.assert_array_equal(w, 1.0)


def test_route_k_equals_E_is_a_full_argsort_and_softmax():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((6, 9)).astype(np.float32)
    ids, w = L.route_topk(logits, 9)
    np.testing.assert_array_equal(ids, np.argsort(-logits.astype(np.float64), axis=1, kind="stable"))
    ref = np.take_along_axis(scipy.special.softmax(logits.astype(np.float64), axis=1), ids.astype(int), 1)
    np.testing.assert_allclose(w, ref, rtol=1e-13)


def test_route_without_renormalization_is_full_softmax():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((6, 32)).astype(np.float32)
    ids, w = L.route_topk(logits, 6, renormalize=False)
    ref = np.take_along_axis(scipy.special.softmax(logits.astype(np.float64), axis=1), ids.astype(int), 1)
    np.testing.assert_allclose(w, ref, rtol=1e-13)
    assert (w.sum(1) < 1).all()


# ------------------------------------------------------ per-token FP8 quant ----
def test_quant_max_element_encodes_to_448_and_error_is_half_ulp():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((40, 512)) * 10.0 ** rng.integers(-3, 3, (40, 1))).astype(np.float32)
    q, s = L.quant_fp8_per_token(x)
    assert s.dtype == np.float32
    amax_idx = np.abs(x).argmax(1)
    top = q[np.arange(40), amax_idx]
    assert set(np.unique(top & 0x7F)) == {0x7E}
    assert ((top >> 7) == (x[np.arange(40), amax_idx] < 0)).all()
    r = (x / s[:, None]).astype(np.float64)
    deq = F.e4m3_decode(q)
    # E4M3 spacing at |r|: 2^(floor(log2|r|) - 3) for normals, 2^-9 below 2^-6
    e = np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -6)))
    ulp = 2.0 ** (e - 3)
    assert (np.abs(r - deq) <= ulp / 2 * (1 + 1e-6)).all()


def test_quant_matches_torch_reference_construction():
    rng = np.random.default_rng(7)
    x = torch.from_numpy(rng.standard_normal((64, 1024)).astype(np.float32)).to(torch.bfloat16)
    xf = x.to(torch.float32)
    s_ref = xf.abs().amax(1) / 448.0
    q_ref = (xf / s_ref[:, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    q, s = L.quant_fp8_per_token(xf.numpy())
    np.testing.assert_array_equal(s, s_ref.numpy())
    np.testing.assert_array_equal(q, q_ref.numpy())


def test_quant_zero_row():
    x = np.zeros((2, 256), dtype=np.float32)
    x[1, 3] = -2.5
    q, s = L.quant_fp8_per_token(x)
    assert s[0] == 0 and (q[0] == 0).all()
    assert q[1, 3] == 0xFE and s[1] == np.float32(2.5) / np.float32(448)


# ------------------------------------------------------------ INT4 g128 ----
def test_int4_quant_brute_force():
    rng = np.random.default_rng(8)
    w = (rng.standard_normal((6, 384)) * 0.02).astype(np.float32)
    w[2, 128:256] = 0.0                               # a zero group
    codes, s = L.quantize_int4_g128(w)
    assert s.shape == (6, 3)
    for r in range(6):
        for g in range(3):
            grp = [float(v) for v in w[r, 128 * g:128 * (g + 1)]]
            a = max(abs(v) for v in grp)
            sc = float(np.float32(a) / np.float32(7.0))
            assert s[r, g] == sc
            for i, v in enumerate(grp):
                want = 0 if sc == 0 else max(-8, min(7, round(float(np.float32(v) / np.float32(sc)))))
                assert codes[r, 128 * g + i] == want      # Python round() is half-to-even


def test_int4_quant_bf16_scales_brute_force():
    # the stored scale is torch's bfloat16 cast of fl32(a / 7); codes against it
    rng = np.random.default_rng(18)
    w = (rng.standard_normal((5, 256)) * 0.02).astype(np.float32)
    w[1, :128] = 0.0                                  # a zero group
    w[3, 5] = 0.02 * 7 * 1.003                        # scale rounded down: |w/s| > 7 -> clamp
    codes, s = L.quantize_int4_g128(w, scale_dtype="bf16")
    for r in range(5):
        for g in range(2):
            grp = [float(v) for v in w[r, 128 * g:128 * (g + 1)]]
            a = max(abs(v) for v in grp)
            sc = float(torch.tensor(float(np.float32(a) / np.float32(7.0)),
                                    dtype=torch.float32).to(torch.bfloat16).float())
            assert s[r, g] == sc
            for i, v in enumerate(grp):
                want = 0 if sc == 0 else max(-8, min(7, round(float(np.float32(v) / np.float32(sc)))))
                assert codes[r, 128 * g + i] == want
    assert np.abs(codes).max() <= 7                   # max/bf16(max/7) stays below 7.5


def test_int4_quant_invariants_and_scale_shape_from_card():
    d = _golden_shapes()
    rows, cols = int(d["proj_rows"]), int(d["proj_cols"])
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    codes, s = L.quantize_int4_g128(w)
    assert s.shape == (int(d["proj_scale_rows"]), int(d["proj_scale_cols"]))
    assert codes.min() >= -8 and codes.max() <= 7
    g = codes.reshape(rows, -1, 128)
    assert (np.abs(g).max(axis=2) == 7).all()        # each group's max element -> +-7
    err = np.abs(w.reshape(rows, -1, 128) - g * s[:, :, None].astype(np.float64))
    assert (err <= s[:, :, None] / 2 * (1 + 1e-6)).all()
    packed, s2 = L.pack_int4_g128(w)
    assert packed.shape == (rows, cols // 2) and (s2 == s).all()


def test_payload_accounting_from_card_fixes_per_expert_shape():
    d = _golden_shapes()
    H, I, E = int(d["hidden"]), int(d["expert_width"]), int(d["routed_experts_per_sparse_layer"])
    P = 3 * H * I                                      # gate, up, down
    routed_i8_gib = d["sparse_layers"] * E * P / 2 ** 30
    assert routed_i8_gib == pytest.approx(240.0)
    assert routed_i8_gib < d["i8_payload_gib"] < routed_i8_gib * 1.02
    assert d["i8_payload_gib"] / 2 + d["bf16_payload_gib"] == pytest.approx(d["packed_payload_gib"], abs=0.01)
    cfg = W.get_config("decode")
    assert (cfg.H, cfg.I, cfg.E, cfg.k) == (H, I, E, int(d["active_experts"]))


# ----------------------------------------------------------------- permute ----
def test_permute_matches_brute_force():
    rng = np.random.default_rng(10)
    for T, k, E in [(16, 2, 8), (9, 6, 256), (33, 3, 5), (1, 1, 4)]:
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        p = L.permute_plan(ids, E)
        flat = ids.reshape(-1)
        sorted_rows = [r for e in range(E) for r in range(T * k) if flat[r] == e]
        assert list(p["sorted_rows"]) == sorted_rows
        counts = [int((flat == e).sum()) for e in range(E)]
        assert list(p["counts"]) == counts
        assert list(p["offsets"]) == [sum(counts[:e]) for e in range(E + 1)]
        for pos, r in enumerate(sorted_rows):
            assert p["row_pos"][r] == pos
        assert list(p["active"]) == [e for e in range(E) if counts[e]]
        xq = rng.integers(0, 255, (T, 4)).astype(np.uint8)
        xs = rng.random(T).astype(np.float32)
        gq, gs = L.gather_rows(xq, xs, p["sorted_rows"], k)
        for pos, r in enumerate(sorted_rows):
            assert (gq[pos] == xq[r // k]).all() and gs[pos] == xs[r // k]


# ------------------------------------------------------------ grouped GEMM ----
def _rand_case(rng, R, N, K, E):
    a_q = F.e4m3_encode(rng.standard_normal((R, K)) * 50)
    a_s = rng.random(R).astype(np.float32) + 0.01
    codes = rng.integers(-8, 8, (E, N, K)).astype(np.int8)
    s_w = (rng.random((E, N, K // 128)) * 0.01).astype(np.float32)
    experts = np.sort(rng.integers(0, E, R))
    return a_q, a_s, codes, s_w, experts


def test_w4a8_equals_dequantize_then_matmul():
    rng = np.random.default_rng(11)
    a_q, a_s, codes, s_w, experts = _rand_case(rng, 20, 48, 384, 3)
    out = L.w4a8_rows(a_q, a_s, experts, lambda e: codes[e], lambda e: s_w[e])
    x_deq = L.dequant_fp8_rows(a_q, a_s)                                   # [R, K]
    for p in range(20):
        e = experts[p]
        w_deq = codes[e].astype(np.float64) * np.repeat(s_w[e].astype(np.float64), 128, axis=1)
        ref = torch.from_numpy(w_deq) @ torch.from_numpy(x_deq[p])        # different library
        np.testing.assert_allclose(out[p], ref.numpy(), rtol=1e-12, atol=1e-300)


def test_w4a8_integer_special_case_exact():
    # unit scales and activation codes that decode to small integers: every
    # output is an integer, computed here with Python ints.
    rng = np.random.default_rng(12)
    int_codes = {v: int(F.e4m3_encode([v])[0]) for v in range(-8, 9)}
    R, N, K = 6, 16, 256
    a_int = rng.integers(-8, 9, (R, K))
    a_q = np.vectorize(int_codes.get)(a_int).astype(np.uint8)
    codes = rng.integers(-8, 8, (1, N, K)).astype(np.int8)
    out = L.w4a8_rows(a_q, np.ones(R, np.float32), np.zeros(R, int),
                      lambda e: codes[e], lambda e: np.ones((N, K // 128), np.float32))
    for p in range(R):
        for n in range(N):
            assert out[p, n] == sum(int(a_int[p, kk]) * int(codes[0, n, kk]) for kk in range(K))


def test_w4a8_one_hot_codes_select_activation_columns():
    rng = np.random.default_rng(13)
    R, N, K = 5, 12, 256
    a_q = F.e4m3_encode(rng.standard_normal((R, K)))
    a_s = rng.random(R).astype(np.float32)
    perm = rng.permutation(K)[:N]
    codes = np.zeros((1, N, K), np.int8)
    codes[0, np.arange(N), perm] = 1
    s_w = rng.random((1, N, 2)).astype(np.float32)
    out = L.w4a8_rows(a_q, a_s, np.zeros(R, int), lambda e: codes[e], lambda e: s_w[e])
    dec = F.e4m3_decode(a_q)
    for n in range(N):
        expect = a_s.astype(np.float64) * s_w[0, n, perm[n] // 128] * dec[:, perm[n]]
        np.testing.assert_array_equal(out[:, n], expect)


def test_fp8row_equals_dequantize_then_matmul_and_row_max():
    rng = np.random.default_rng(14)
    w = (rng.standard_normal((2, 24, 256)) * 0.02).astype(np.float32)
    wq, srow = zip(*[L.quant_fp8_per_row_weights(w[e]) for e in range(2)])
    for e in range(2):
        top = wq[e][np.arange(24), np.abs(w[e]).argmax(1)]
        assert set(np.unique(top & 0x7F)) == {0x7E}
    a_q = F.e4m3_encode(rng.standard_normal((7, 256)) * 30)
    a_s = rng.random(7).astype(np.float32)
    experts = np.array([0, 0, 1, 1, 1, 0, 1])
    out = L.fp8row_rows(a_q, a_s, experts, lambda e: wq[e], lambda e: srow[e])
    for p in range(7):
        e = experts[p]
        w_deq = F.e4m3_decode(wq[e]) * srow[e].astype(np.float64)[:, None]
        ref = sum(w_deq[:, kk] * (F.e4m3_decode(a_q[p, kk:kk + 1])[0] * float(a_s[p])) for kk in range(256))
        np.testing.assert_allclose(out[p], ref, rtol=1e-12)


# ----------------------------------------------------------- SwiGLU, combine ----
def test_requant_fnuz_hand_example():
    # row [0x7F, 0x01, 0x80, 0xC8] with s = 0.5: FNUZ values 240, 2^-10, NaN
    # (read as 0), -2 -> w = [120, 2^-11, 0, -1]; s' = 120/448; w/s' = 448,
    # 0.0018 (nearest E4M3: 2^-9 = 0x01), 0, -3.733 (nearest: -3.75 = 0xC7)
    q, s = L.requant_fnuz_rows(np.array([[0x7F, 0x01, 0x80, 0xC8]], dtype=np.uint8),
                               np.array([0.5], dtype=np.float32))
    assert q.tolist() == [[0x7E, 0x01, 0x00, 0xC7]]
    assert s[0] == np.float32(np.float32(120.0) / np.float32(448.0))


def test_requant_fnuz_matches_library_composition():
    # the same steps with library routines: torch's FNUZ decode, numpy float32
    # products and quotients, torch's OCP cast (RNE; magnitudes stay <= 448)
    rng = np.random.default_rng(11)
    b = rng.integers(0, 256, size=(24, 256), dtype=np.uint8)
    b[b == 0x80] = 0x00
    b[:, 7] = 0x7F                                         # every row has a max element
    s = (rng.random(24) * 1e-2 + 1e-4).astype(np.float32)
    q, s2 = L.requant_fnuz_rows(b, s)
    v = torch.from_numpy(b).view(torch.float8_e4m3fnuz).to(torch.float32).numpy()
    w = s[:, None] * v
    s_ref = (np.abs(w).max(axis=1) / np.float32(448.0)).astype(np.float32)
    ratio = (w / s_ref[:, None]).astype(np.float32)
    q_ref = torch.from_numpy(ratio).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(s2, s_ref)
    assert np.array_equal(q, q_ref)
    assert np.all(q[:, 7] == 0x7E)                         # the row max encodes to 448


def test_requant_fnuz_error_bound():
    # each requantized element is within half an E4M3 step of the FNUZ value
    rng = np.random.default_rng(12)
    b = rng.integers(0, 256, size=(16, 512), dtype=np.uint8)
    b[b == 0x80] = 0x00
    s = np.full(16, 3e-3, dtype=np.float32)
    q, s2 = L.requant_fnuz_rows(b, s)
    w = s[:, None].astype(np.float64) * F.e4m3fnuz_decode(b)
    back = F.e4m3_decode(q) * s2[:, None].astype(np.float64)
    # E4M3 relative step 2^-3 for normals; absolute 2^-9 s' below 2^-6 s'
    bound = np.maximum(np.abs(w) * 2.0 ** -4, 2.0 ** -10 * s2[:, None]) * (1 + 1e-6)
    assert np.all(np.abs(back - w) <= bound)


def test_nvfp4_dequant_hand_example():
    # one row of 32 codes: block 0 scale 0x38 (1.0), block 1 scale 0x41 (2.25),
    # scale2 0.5: W = LUT[c] * block scale * 0.5
    codes = np.array([[1, 7, 15, 0] + [4] * 12 + [3, 9] + [2] * 14], dtype=np.uint8)
    w = L.nvfp4_dequant(F.pack_fp4(codes), np.array([[0x38, 0x41]], dtype=np.uint8), 0.5)
    assert w[0, :4].tolist() == [0.25, 3.0, -3.0, 0.0]
    assert w[0, 4] == 1.0                             # code 4 = 2.0 -> 2 * 1 * 0.5
    assert w[0, 16] == 1.5 * 2.25 * 0.5 and w[0, 17] == -0.5 * 2.25 * 0.5
    assert w[0, 18] == 1.0 * 2.25 * 0.5


def test_nvfp4_rows_brute_force():
    rng = np.random.default_rng(32)
    E, N, K, R = 2, 3, 32, 4
    codes = rng.integers(0, 16, (E, N, K)).astype(np.uint8)
    bs = rng.integers(0x28, 0x48, (E, N, K // 16)).astype(np.uint8)
    s2 = np.array([0.25, 0.125], dtype=np.float32)
    a_q = F.e4m3_encode(rng.standard_normal((R, K)))
    a_s = np.array([1.0, 0.5, 2.0, 0.75], dtype=np.float32)
    experts = np.array([0, 0, 1, 1])
    got = L.nvfp4_rows(a_q, a_s, experts, lambda e: F.pack_fp4(codes[e]), lambda e: bs[e],
                       lambda e: s2[e])
    tab = [0, .5, 1, 1.5, 2, 3, 4, 6]
    for p in range(R):
        e = experts[p]
        for n in range(N):
            acc = 0.0
            for k in range(K):
                c = int(codes[e, n, k])
                wv = (-1 if c >= 8 else 1) * tab[c & 7] * float(F.e4m3_decode([bs[e, n, k // 16]])[0])
                acc += float(F.e4m3_decode([a_q[p, k]])[0]) * wv
            assert got[p, n] == pytest.approx(float(a_s[p]) * float(s2[e]) * acc, rel=1e-12, abs=1e-300)


def test_aqlm_dequant_hand_example_and_int16_wrap():
    # two books: a 65536-entry book addressed by int16 codes (negative values wrap
    # to idx & 0xFFFF) and a 256-entry book addressed by uint8 codes
    b0 = np.zeros((65536, 8), np.float16)
    b0[5] = np.arange(8, dtype=np.float16)               # 0..7
    b0[0xFFFE] = np.float16(0.5)                         # reached by int16 code -2
    b1 = np.zeros((256, 8), np.float16)
    b1[3] = np.float16(-1.0)
    codes0 = np.array([[5, -2]], dtype=np.int16)
    codes1 = np.array([[3, 0]], dtype=np.uint8)
    w = L.aqlm_dequant([codes0, codes1], [b0, b1], np.array([2.0], np.float16))
    assert w[0, :8].tolist() == [2.0 * (i - 1.0) for i in range(8)]
    assert w[0, 8:].tolist() == [1.0] * 8


def test_aqlm_rows_brute_force():
    rng = np.random.default_rng(33)
    E, N, K, R = 2, 3, 32, 4
    b0 = rng.standard_normal((300, 8)).astype(np.float16)
    codes = rng.integers(0, 300, (E, N, K // 8)).astype(np.int16)
    sc = (rng.random((E, N)) + 0.5).astype(np.float16)
    a_q = F.e4m3_encode(rng.standard_normal((R, K)))
    a_s = np.array([1.0, 0.5, 2.0, 0.75], dtype=np.float32)
    experts = np.array([0, 1, 1, 0])
    got = L.aqlm_rows(a_q, a_s, experts, lambda e: [codes[e]], [b0], lambda e: sc[e])
    for p in range(R):
        e = experts[p]
        for n in range(N):
            acc = 0.0
            for k in range(K):
                wv = float(b0[codes[e, n, k // 8], k % 8]) * float(sc[e, n])
                acc += float(F.e4m3_decode([a_q[p, k]])[0]) * wv
            assert got[p, n] == pytest.approx(float(a_s[p]) * acc, rel=1e-12, abs=1e-300)


def test_silu_closed_forms():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(L.silu(z), z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)
    assert L.silu(np.array([0.0]))[0] == 0.0
    assert abs(L.silu(np.array([40.0]))[0] - 40.0) < 1e-15
    o13 = np.array([[1.0, -2.0, 3.0, 5.0]])            # gate = [1, -2], up = [3, 5]
    h = L.silu_mul(o13)
    expect = [1.0 / (1 + np.exp(-1.0)) * 3.0, -2.0 / (1 + np.exp(2.0)) * 5.0]
    np.testing.assert_array_equal(h[0], F.bf16_round(expect))


def test_combine_brute_force_and_special_cases():
    rng = np.random.default_rng(15)
    T, k, E, H = 6, 3, 5, 16
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    p = L.permute_plan(ids, E)
    o = F.bf16_round(rng.standard_normal((T * k, H)))
    w = rng.random((T, k))
    sh = F.bf16_round(rng.standard_normal((T, H)))
    y = L.combine(o, p["row_pos"], w, k, sh)
    for t in range(T):
        for c in range(H):
            acc = 0.0
            for j in range(k):
                acc += w[t, j] * o[p["row_pos"][t * k + j], c]
            assert y[t, c] == F.bf16_round([acc + sh[t, c]])[0]
    # k = 1 with weight 1 returns the expert output unchanged
    ids1 = rng.integers(0, E, (T, 1))
    p1 = L.permute_plan(ids1, E)
    o1 = F.bf16_round(rng.standard_normal((T, H)))
    y1 = L.combine(o1, p1["row_pos"], np.ones((T, 1)), 1)
    np.testing.assert_array_equal(y1, o1[p1["row_pos"]])


def test_shared_mlp_fused_equals_sum_of_two_and_torch():
    cfg = W.get_config("tiny", n_shared=2, I=128)
    ws13, ws2 = W.make_shared_weights(cfg)
    x = W.make_activations(cfg).to(torch.bfloat16)
    y = L.shared_mlp(x.float().numpy(), ws13.float().numpy(), ws2.float().numpy())
    # the two experts separately, in torch float64, summed before the final rounding
    xd = x.double()
    I = cfg.I
    acc = torch.zeros(cfg.T, cfg.H, dtype=torch.float64)
    for j in range(2):
        g = ws13[j * I:(j + 1) * I].double()
        u = ws13[2 * I + j * I:2 * I + (j + 1) * I].double()
        d = ws2[:, j * I:(j + 1) * I].double()
        h = torch.nn.functional.silu(xd @ g.T) * (xd @ u.T)
        h = torch.from_numpy(F.bf16_round(h.numpy()))
        acc += h @ d.T
    np.testing.assert_allclose(y, F.bf16_round(acc.numpy()), rtol=0, atol=0)


# ------------------------------------------------------------- whole layer ----
def _tiny_layer(cfg):
    inp = W.make_layer_inputs(cfg)
    x = inp["x"].float().numpy()
    res = L.moe_layer(x, inp["logits"].numpy(), cfg.k, w13=inp["w13"].numpy(),
                      w2=inp["w2"].numpy(), bias=None if inp["bias"] is None else inp["bias"].numpy())
    return inp, res


def _deq_int4(w):
    c, s = L.quantize_int4_g128(w)
    return c * np.repeat(s.astype(np.float64), 128, axis=1)


def test_layer_close_to_loop_reference_with_dequantized_weights():
    # A per-token Python-loop evaluation with the INT4-dequantized weights and
    # unquantized activations differs from the oracle only by the FP8 activation
    # rounding (a few percent); a dropped term or wrong index would be far off.
    cfg = W.get_config("tiny")
    inp, res = _tiny_layer(cfg)
    x, lg = inp["x"].float().numpy(), inp["logits"].numpy()
    w13, w2 = inp["w13"].numpy(), inp["w2"].numpy()
    deq13 = np.stack([_deq_int4(w13[e]) for e in range(cfg.E)])
    deq2 = np.stack([_deq_int4(w2[e]) for e in range(cfg.E)])
    ref = L.unquantized_layer(x, lg, cfg.k, deq13, deq2)
    rel = np.linalg.norm(res["y"] - ref) / np.linalg.norm(ref)
    assert rel < 0.08, rel
    # against full-precision weights the INT4 error dominates (~20 %): sanity only
    ref_fp = L.unquantized_layer(x, lg, cfg.k, w13, w2)
    assert np.linalg.norm(res["y"] - ref_fp) / np.linalg.norm(ref_fp) < 0.35
    assert res["y"].shape == (cfg.T, cfg.H) and np.isfinite(res["y"]).all()


def test_layer_single_expert_is_a_dense_quantized_mlp():
    cfg = W.get_config("tiny", E=1, k=1)
    inp, res = _tiny_layer(cfg)
    assert (res["topk_ids"] == 0).all() and (res["topk_w"] == 1).all()
    x = inp["x"].float().numpy()
    xq, xs = L.quant_fp8_per_token(x)
    w13, w2 = inp["w13"][0].numpy(), inp["w2"][0].numpy()
    c13, s13 = L.quantize_int4_g128(w13)
    c2, s2 = L.quantize_int4_g128(w2)
    # dense evaluation with dequantized operands (a different association)
    g13 = L.dequant_fp8_rows(xq, xs) @ (c13 * np.repeat(s13.astype(np.float64), 128, 1)).T
    h = L.silu_mul(g13)
    hq, hs = L.quant_fp8_per_token(h)
    o = F.bf16_round(L.dequant_fp8_rows(hq, hs) @ (c2 * np.repeat(s2.astype(np.float64), 128, 1)).T)
    np.testing.assert_allclose(res["y"], o, rtol=2 ** -7, atol=0)
    assert np.mean(res["y"] == o) > 0.99


def test_layer_fp8row_variant_runs_and_is_close():
    cfg = W.get_config("tiny", weight_format="fp8row")
    inp = W.make_layer_inputs(cfg)
    res = L.moe_layer(inp["x"].float().numpy(), inp["logits"].numpy(), cfg.k,
                      w13=inp["w13"].numpy(), w2=inp["w2"].numpy(), fp8row=True)
    ref = L.unquantized_layer(inp["x"].float().numpy(), inp["logits"].numpy(), cfg.k,
                              inp["w13"].numpy(), inp["w2"].numpy())
    assert np.linalg.norm(res["y"] - ref) / np.linalg.norm(ref) < 0.1
