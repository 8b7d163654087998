"""Plain CPU oracle of the KV write path: quantising new global-KV entries and the
sliding-window rows.  TEST INFRASTRUCTURE.

The pages fix the sizes, not the encoders: "DeepSeek-V4.1 模型结构（0）：一张图看懂
DeepSeek-V4.1-Flash", Q&A on how the 890-byte figure is derived (a main entry is 512
4-bit values plus 32 bytes of scale, an indexer entry 128 4-bit values plus a 4-byte
scale), and "DeepSeek V4.1 Flash 深度解析", part 4 entry on FP4 in the KV cache (the main
KV and the indexer use different 4-bit formats; the sliding window stays FP8).

Readings taken (also listed in the design notes):
  Q1  indexer entry: scale = fl32(amax / 6) over the 128 values (1 when that is below
      the smallest normal fp32, 2^-126); code_d = E2M1 of fl32(x_d / scale).
  Q2  main entry: per group of 16 values, scale = E4M3 of fl32(amax / 6) (nearest, ties
      to even, saturating at 448; the zero code becomes code 1, 2^-9);
      code_d = E2M1 of fl32(x_d / scale).
  Q3  E2M1 of a value: the nearest of the 16 codes, ties to the code with mantissa bit 0,
      magnitudes above 6 saturate to 6; the sign bit is the input's sign bit (so -0 and
      small negatives give code 8).
  Q4  a window row is the E4M3 (nearest, ties to even, saturating at 448) of each bf16
      value; the row for position p lives in ring slot p mod 128.
  Q5  element 2i of a row sits in the low nibble of byte i.

Each encoder is written as "nearest representable value" over the decoded code table,
the definition of round-to-nearest, rather than as bit manipulation.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_decode, e2m1_decode, e4m3_decode

D_IDX = 128
D_KV = 512
SWA_W = 128
SCALE_GROUP = 16
E4M3_MAX_CODE = 0x7E          # 448, the largest finite E4M3 value
FP32_MIN_NORMAL = 2.0 ** -126


def _f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32)


def _nearest_code(a: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the entry of the ascending non-negative `table` nearest to each |a| value,
    ties to the even index (= mantissa bit 0 for the code tables used here), values past
    the end saturating to the last entry."""
    a = np.asarray(a, dtype=np.float64)
    hi = np.searchsorted(table, a, side="left")          # first table value >= a
    hi = np.clip(hi, 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    d_lo = np.abs(a - table[lo])
    d_hi = np.abs(table[hi] - a)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    # at or past the largest value: saturate (for huge values the two fp64 distances are
    # equal and the tie rule above would pick the lower neighbour)
    return np.where(a >= table[-1], len(table) - 1, np.where(pick_hi, hi, lo))


_E2M1_MAG = e2m1_decode(np.arange(8))                    # 0, .5, 1, 1.5, 2, 3, 4, 6
_E4M3_MAG = e4m3_decode(np.arange(E4M3_MAX_CODE + 1))    # codes 0x00..0x7E, ascending


def e2m1_encode(q: np.ndarray) -> np.ndarray:
    """fp32 values -> 4-bit E2M1 codes (reading Q3)."""
    q = _f32(q)
    mag = _nearest_code(np.abs(q.astype(np.float64)), _E2M1_MAG).astype(np.uint8)
    return mag | (np.signbit(q).astype(np.uint8) << 3)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Finite values -> E4M3 bytes, nearest with ties to even, saturating at +-448."""
    v = np.asarray(v, dtype=np.float64)
    mag = _nearest_code(np.abs(v), _E4M3_MAG).astype(np.uint8)
    return mag | (np.signbit(v).astype(np.uint8) << 7)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., 2n] codes -> [..., n] bytes, element 2i in the low nibble (reading Q5)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def quantize_index_entry(x_bits: np.ndarray):
    """bf16 [n, 128] -> (codes u8 [n, 64], scale f32 [n]) (reading Q1)."""
    x = _f32(bf16_decode(x_bits))
    amax = np.abs(x).max(axis=-1)
    scale = amax / np.float32(6.0)                       # fp32 division, nearest-even
    scale = np.where(scale >= np.float32(FP32_MIN_NORMAL), scale, np.float32(1.0)).astype(np.float32)
    q = x / scale[:, None]                               # fp32 division, nearest-even
    return pack_nibbles(e2m1_encode(q)), scale


def quantize_main_entry(x_bits: np.ndarray):
    """bf16 [n, 512] -> (codes u8 [n, 256], scale bytes u8 [n, 32] E4M3) (reading Q2)."""
    x = _f32(bf16_decode(x_bits))
    n = x.shape[0]
    g = x.reshape(n, D_KV // SCALE_GROUP, SCALE_GROUP)
    amax = np.abs(g).max(axis=-1)
    t = amax / np.float32(6.0)                           # fp32 division, nearest-even
    s_code = e4m3_encode(t)
    s_code = np.where(s_code == 0, np.uint8(1), s_code).astype(np.uint8)
    s = _f32(e4m3_decode(s_code))
    q = g / s[..., None]                                 # fp32 division, nearest-even
    codes = e2m1_encode(q).reshape(n, D_KV)
    return pack_nibbles(codes), s_code


def swa_encode(x_bits: np.ndarray) -> np.ndarray:
    """bf16 [..., 512] -> E4M3 bytes [..., 512] (reading Q4)."""
    return e4m3_encode(bf16_decode(x_bits))


def kv_append(idx_codes, idx_scale, kv_codes, kv_scale, x_idx_bits, x_kv_bits, dst):
    """Quantise rows i of x_idx / x_kv into entry dst[i] of copies of the four planes.
    Rows whose dst lies outside [0, capacity) are not written; returns the new planes and
    the number of such rows.  dst ids are distinct."""
    idx_codes, idx_scale = idx_codes.copy(), idx_scale.copy()
    kv_codes, kv_scale = kv_codes.copy(), kv_scale.copy()
    cap = idx_codes.shape[0]
    dst = np.asarray(dst, dtype=np.int64)
    ok = (dst >= 0) & (dst < cap)
    ic, isc = quantize_index_entry(np.asarray(x_idx_bits)[ok])
    kc, ksc = quantize_main_entry(np.asarray(x_kv_bits)[ok])
    idx_codes[dst[ok]] = ic
    idx_scale[dst[ok]] = isc
    kv_codes[dst[ok]] = kc
    kv_scale[dst[ok]] = ksc
    return idx_codes, idx_scale, kv_codes, kv_scale, int((~ok).sum())


def swa_append(swa: np.ndarray, x_bits: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Write E4M3(x[b]) into ring slot pos[b] mod 128 of a copy of swa [B][128][512];
    sequences with pos < 0 are left alone."""
    swa = swa.copy()
    for b, p in enumerate(np.asarray(pos, dtype=np.int64)):
        if p >= 0:
            swa[b, p % SWA_W] = swa_encode(np.asarray(x_bits)[b])
    return swa
