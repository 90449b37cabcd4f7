"""Narrow storage formats used by the layer -- oracle side (test infrastructure).

* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
  infinities; 0x7F/0xFF are NaN; largest finite magnitude 448.  The row-FP8
  card ("Inkling 2 Small FP8 for AMD MI300X", "Precision and files") uses the
  FNUZ flavour with max 240 on MI300X; the flavour native to gfx950 is OCP, so
  the divisor used throughout is 448 (reading recorded in the design notes).
* E4M3FNUZ (the MI300X flavour of the row-FP8 card): 1 sign, 4 exponent
  (bias 8), 3 mantissa bits; no infinities and no negative zero; 0x80 is the
  only NaN; largest finite magnitude 240 (0x7F).  Read only, to convert such
  checkpoints to OCP E4M3.
* E2M1 (FP4, the NVFP4 element format of the hot experts in
  "Inkling-512k-NVFP4-AQLM-hybrid", "Dequant math"): the 16 codes decode to
  [0, .5, 1, 1.5, 2, 3, 4, 6, -0, -.5, -1, -1.5, -2, -3, -4, -6]; two codes per
  byte, the low nibble first.
* bfloat16: the top 16 bits of an IEEE binary32.
* INT4: signed codes in [-8, 7] stored as nibble = code + 8, eight consecutive
  codes per little-endian 32-bit word with the first code in the least
  significant nibble ("wstewart3/Inkling-Small-W4A8-G128", §7 "Recover and
  physically pack INT4", packing bullets).  Viewed as bytes this is two codes
  per byte, first code in the low nibble.  The kernels read these bytes in a
  tiled order of their own (tile_int4), a permutation of whole bytes.

Rounding is round-to-nearest-even everywhere (the pages do not name a rounding
mode; RNE is the IEEE default).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN_CODES = (0x7F, 0xFF)


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 byte, as float64 (NaN for 0x7F / 0xFF).

    normal (exponent field e >= 1): (-1)^s * 2^(e-7) * (1 + m/8)
    subnormal (e == 0):             (-1)^s * 2^(-6) * (m/8)
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where(s == 1, -mag, mag)
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return val.astype(np.float64)


# all 127 non-negative finite values, indexed by their code 0x00..0x7E (ascending)
_E4M3_POS = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def _e4m3_encode_block(v):
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")          # first table value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    exact = _E4M3_POS[hi] == a
    pick_hi = exact | (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def e4m3_encode(v, block: int = 1 << 19) -> np.ndarray:
    """Nearest E4M3 code to each finite value, ties to the even code, saturating.

    The representable non-negative values in increasing order have increasing
    codes 0x00..0x7E, and the least significant code bit is the least significant
    mantissa bit, so "ties to even" means "ties to the even code".  Magnitudes at
    or above 448 saturate to 448 (0x7E) because E4M3 has no infinity.  The sign
    bit is kept, so a negative value that rounds to zero encodes as 0x80.
    (Values are processed in blocks only to bound temporary memory.)
    """
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("e4m3_encode: NaN input")
    flat = v.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for i in range(0, flat.size, block):
        out[i:i + block] = _e4m3_encode_block(flat[i:i + block])
    return out.reshape(v.shape)


def e4m3fnuz_decode(codes) -> np.ndarray:
    """Value of each E4M3FNUZ byte, as float64 (NaN for 0x80).

    normal (exponent field e >= 1): (-1)^s * 2^(e-8) * (1 + m/8)
    subnormal (e == 0):             (-1)^s * 2^(-7) * (m/8)
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -7), np.ldexp(1.0 + m / 8.0, e - 8))
    val = np.where(s == 1, -mag, mag)
    val = np.where(c == 0x80, np.nan, val)
    return val.astype(np.float64)


E2M1_VALUES = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6],
                       dtype=np.float64)


def e2m1_decode(codes) -> np.ndarray:
    """Value of each 4-bit E2M1 code 0..15 (float64), by the card's table."""
    return E2M1_VALUES[np.asarray(codes, dtype=np.int64) & 0xF]


def unpack_fp4(packed) -> np.ndarray:
    """Bytes [..., K/2] -> codes [..., K], low nibble first (the card's order)."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def pack_fp4(codes) -> np.ndarray:
    """Codes [..., K] (0..15) -> bytes [..., K/2], the first code in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    if c.shape[-1] % 2 or (c > 15).any():
        raise ValueError("codes must be 0..15 with an even count")
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def fp32(v) -> np.ndarray:
    """Round to IEEE binary32 (RNE) and return as float64."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_round(v) -> np.ndarray:
    """Round float64 values to the bfloat16 grid, RNE, in one step (no double rounding).

    v = m * 2^e with 0.5 <= |m| < 1; bfloat16 keeps 8 significant bits, so the
    result is rint(m * 2^8) * 2^(e-8).  (Overflow and subnormals do not occur for
    the magnitudes this layer produces.)
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def bf16_bits(v) -> np.ndarray:
    """uint16 bit pattern of values already on the bfloat16 grid."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(u) -> np.ndarray:
    u = np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------- INT4
INT4_MIN, INT4_MAX = -8, 7
GROUP = 128


def pack_int4(codes) -> np.ndarray:
    """Codes int [..., K] in [-8, 7] -> bytes uint8 [..., K/2].

    nibble = code + 8; byte b holds codes 2b (low nibble) and 2b+1 (high nibble),
    which is the little-endian byte view of eight codes per 32-bit word with the
    first code in the least significant nibble.
    """
    c = np.asarray(codes)
    if c.shape[-1] % 2:
        raise ValueError("pack_int4: K must be even")
    if (c < INT4_MIN).any() or (c > INT4_MAX).any():
        raise ValueError("pack_int4: code outside [-8, 7]")
    nib = (c.astype(np.int64) + 8).astype(np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed) -> np.ndarray:
    """Bytes uint8 [..., K/2] -> codes int8 [..., K] (inverse of pack_int4)."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0xF).astype(np.int8) - 8
    hi = (p >> 4).astype(np.int8) - 8
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


TILE_ROWS = 16


def tile_int4(packed) -> np.ndarray:
    """Packed INT4 bytes [..., N, K/2] -> the kernels' tiled order
    [..., N/16, K/128, 16, 64]: 16-row blocks, each stored group after group, so
    the 64 bytes (128 codes) of one 128-wide K group of 16 consecutive rows are
    1024 contiguous bytes.  Element [..., b, g, r, c] is byte c of group g of row
    16 b + r, i.e. packed[..., 16 b + r, 64 g + c].  This storage order is the
    library's own (the pages' checkpoints keep rows contiguous); it changes where
    bytes sit, never a byte.
    """
    p = np.asarray(packed, dtype=np.uint8)
    N, K2 = p.shape[-2], p.shape[-1]
    if N % TILE_ROWS or (2 * K2) % GROUP:
        raise ValueError("tile_int4: N must be a multiple of 16 and K of 128")
    lead = p.shape[:-2]
    blocks = p.reshape(lead + (N // TILE_ROWS, TILE_ROWS, (2 * K2) // GROUP, GROUP // 2))
    return np.ascontiguousarray(np.swapaxes(blocks, -3, -2))


def int32_words(packed) -> np.ndarray:
    """Little-endian 32-bit words of packed INT4 bytes ([..., K/2] -> [..., K/8])."""
    p = np.ascontiguousarray(np.asarray(packed, dtype=np.uint8))
    return p.view("<u4").astype(np.uint32)
