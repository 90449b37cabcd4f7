"""Pins for oracle/formats.py: E4M3, bfloat16 and INT4 storage formats.

Each pin checks the oracle against something other than itself: the OCP FP8
definition's fixed points, torch's library casts, hand-derived examples of the
packing rule on the Inkling-Small W4A8 card (section 7), and brute force.
"""
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- E4M3 ----
def test_e4m3_decode_fixed_points():
    # OCP 8-bit floating point specification, E4M3 column: bias 7, max 448,
    # min normal 2^-6, min subnormal 2^-9, S.1111.111 is NaN.
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
             0x38: 1.0, 0x39: 1.125, 0x40: 2.0, 0x44: 3.0, 0x48: 4.0, 0x50: 8.0,
             0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0, 0x7D: 416.0}
    for c, v in cases.items():
        assert F.e4m3_decode([c])[0] == v, hex(c)
    assert np.isnan(F.e4m3_decode([0x7F])[0]) and np.isnan(F.e4m3_decode([0xFF])[0])
    z = F.e4m3_decode([0x80])[0]
    assert z == 0.0 and np.signbit(z)


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_e4m3fnuz_decode_fixed_points():
    # E4M3FNUZ: bias 8, max 240 at S.1111.111, min normal 2^-7, min subnormal
    # 2^-10, 0x80 (the negative-zero pattern) is the only NaN.
    cases = {0x00: 0.0, 0x01: 2.0 ** -10, 0x07: 7 * 2.0 ** -10, 0x08: 2.0 ** -7,
             0x40: 1.0, 0x41: 1.125, 0x48: 2.0, 0x7F: 240.0, 0xFF: -240.0, 0xC0: -1.0,
             0x7E: 224.0}
    for c, v in cases.items():
        assert F.e4m3fnuz_decode([c])[0] == v, hex(c)
    assert np.isnan(F.e4m3fnuz_decode([0x80])[0])


def test_e4m3fnuz_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3fnuz_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fnuz).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_e4m3fnuz_is_half_of_ocp_on_shared_finite_codes():
    # the two flavours differ only in the exponent bias (8 vs 7) and the special
    # codes: a byte that is finite in both decodes to half the OCP value
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], dtype=np.uint8)
    assert np.array_equal(F.e4m3fnuz_decode(codes) * 2.0, F.e4m3_decode(codes))


def test_e2m1_table_matches_the_format_definition():
    # E2M1 (OCP microscaling formats): 1 sign, 2 exponent bits (bias 1), 1 mantissa
    # bit; normal 2^(e-1) (1 + m/2), subnormal (e = 0) m/2 -- independent of the
    # card's table that the oracle uses
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        v = 2.0 ** (e - 1) * (1 + m / 2) if e else m / 2
        v = -v if s else v
        got = F.e2m1_decode([c])[0]
        assert got == v and np.signbit(got) == bool(s), c


def test_fp4_packing_low_nibble_first():
    # the hybrid card's packing puts the earlier weight of each byte's pair in bits 0-3
    assert F.unpack_fp4(np.array([[0x21, 0xF8]], dtype=np.uint8)).tolist() == [[1, 2, 8, 15]]
    rng = np.random.default_rng(31)
    c = rng.integers(0, 16, (5, 64)).astype(np.uint8)
    assert np.array_equal(F.unpack_fp4(F.pack_fp4(c)), c)
    with pytest.raises(ValueError):
        F.pack_fp4(np.array([16, 0], dtype=np.uint8))


def test_e4m3_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert len(codes) == 254
    np.testing.assert_array_equal(F.e4m3_encode(F.e4m3_decode(codes)), codes)


def test_e4m3_encode_ties_and_saturation():
    cases = [
        (1.0625, 0x38),        # midpoint of 1.0 (0x38) and 1.125 (0x39) -> even code
        (1.1875, 0x3A),        # midpoint of 1.125 (0x39) and 1.25 (0x3A) -> even code
        (3 * 2.0 ** -10, 0x02),  # subnormal midpoint of 0x01 and 0x02 -> even
        (2.0 ** -10, 0x00),    # half of the smallest subnormal -> 0 (even)
        (1.5 * 2.0 ** -9, 0x02),  # midpoint 0x01/0x02
        (432.0, 0x7E),         # midpoint of 416 (0x7D) and 448 (0x7E) -> even 0x7E
        (424.0, 0x7D), (440.0, 0x7E),
        (448.0, 0x7E), (464.0, 0x7E), (1e6, 0x7E),   # saturation, no infinity
        (-448.5, 0xFE), (-1e-30, 0x80), (-0.0, 0x80),
    ]
    for v, c in cases:
        assert F.e4m3_encode([v])[0] == c, (v, hex(c), hex(F.e4m3_encode([v])[0]))


def test_e4m3_encode_matches_torch_cast():
    # torch's CPU cast to float8_e4m3fn rounds to nearest even; it returns NaN
    # from 480 up (no saturation), so compare only in [-448, 448].
    rng = np.random.default_rng(0)
    v = rng.standard_normal(200_000).astype(np.float32) * rng.choice(
        [1e-3, 1e-2, 0.1, 1, 10, 100], 200_000).astype(np.float32)
    v = np.clip(v, -448, 448)
    # every midpoint between neighbouring finite codes, and its fp32 neighbours
    pos = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    around = np.concatenate([mids, np.nextafter(mids, np.float32(0)),
                             np.nextafter(mids, np.float32(1e9))])
    v = np.concatenate([v, around, -around, pos.astype(np.float32)])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(F.e4m3_encode(v), ref)


# -------------------------------------------------------------- bfloat16 ----
def test_bf16_round_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(100_000) * 10.0 ** rng.integers(-6, 6, 100_000)).astype(np.float32)
    # exact ties: fp32 values whose low 16 bits are 0x8000
    ties = (rng.integers(0x3F000000, 0x47000000, 1000).astype(np.uint32) & 0xFFFF0000) | 0x8000
    v = np.concatenate([v, ties.view(np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(F.bf16_round(v.astype(np.float64)), ref)


def test_bf16_round_is_a_single_rounding():
    # 1 + 2^-8 + 2^-30: rounding to fp32 first would give the exact tie 1 + 2^-8,
    # which RNE then sends to 1.0; the correct single rounding is 1 + 2^-7.
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert F.bf16_round([v])[0] == 1.0 + 2.0 ** -7
    assert F.bf16_round([1.0 + 2.0 ** -8])[0] == 1.0
    assert F.bf16_round([1.0 + 3 * 2.0 ** -8])[0] == 1.0 + 2.0 ** -6


def test_bf16_bits_roundtrip():
    u = np.arange(0, 65536, 7, dtype=np.uint16)
    u = u[((u >> 7) & 0xFF) != 0xFF]    # drop inf/nan
    np.testing.assert_array_equal(F.bf16_bits(F.bf16_from_bits(u)), u)


# ------------------------------------------------------------------ INT4 ----
def _golden_pack_rows():
    rows = []
    with open(os.path.join(GOLDEN, "int4_pack_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            codes, word, byts = [p.strip() for p in line.split(";")]
            rows.append(([int(c) for c in codes.split()], int(word, 16),
                         [int(b, 16) for b in byts.split()]))
    return rows


def test_int4_pack_golden_examples():
    rows = _golden_pack_rows()
    assert len(rows) >= 5
    for codes, word, byts in rows:
        packed = F.pack_int4(np.array([codes], dtype=np.int8))
        assert list(packed[0]) == byts
        assert int(F.int32_words(packed)[0, 0]) == word
        np.testing.assert_array_equal(F.unpack_int4(packed)[0], codes)


def test_int4_pack_brute_force_and_roundtrip():
    rng = np.random.default_rng(2)
    codes = rng.integers(-8, 8, size=(5, 256)).astype(np.int8)
    packed = F.pack_int4(codes)
    assert packed.shape == (5, 128)
    words = F.int32_words(packed)
    for r in range(5):
        for w in range(32):
            expect = 0
            for i in range(8):                       # first code in the LS nibble
                expect |= (int(codes[r, 8 * w + i]) + 8) << (4 * i)
            assert int(words[r, w]) == expect
    np.testing.assert_array_equal(F.unpack_int4(packed), codes)


def test_tile_int4_brute_force():
    """Every byte of the tiled order lands at the offset its definition gives:
    ((b * G + g) * 16 + r) * 64 + c for byte c of group g of row 16 b + r, per
    expert; a pure permutation (sorting recovers the input)."""
    rng = np.random.default_rng(3)
    E, N, K = 2, 48, 384
    G = K // 128
    packed = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    tiled = F.tile_int4(packed)
    assert tiled.shape == (E, N // 16, G, 16, 64)
    flat = tiled.reshape(E, -1)
    for e in range(E):
        for n in range(N):
            for kb in range(K // 2):
                b, r, g, c = n // 16, n % 16, kb // 64, kb % 64
                assert flat[e, ((b * G + g) * 16 + r) * 64 + c] == packed[e, n, kb]
    np.testing.assert_array_equal(np.sort(flat, axis=1), np.sort(packed.reshape(E, -1), axis=1))
    with pytest.raises(ValueError):
        F.tile_int4(packed[:, :40])


def test_int4_pack_rejects_out_of_range():
    with pytest.raises(ValueError):
        F.pack_int4(np.array([[8, 0]]))
    with pytest.raises(ValueError):
        F.pack_int4(np.array([[-9, 0]]))
