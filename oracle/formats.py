"""Number-format decoders for the oracle (fp64, numpy).  TEST INFRASTRUCTURE.

Each decoder is written from the format's definition, bit by bit, so that it
can be checked against independent sources (the OCP table, torch's float8 and
bfloat16 casts) by the pins under tests/.

Formats (a reading of "DeepSeek-V4.1 模型结构（0）：一张图看懂 DeepSeek-V4.1-Flash",
Q&A on the 890-byte count, which fixes only "4-bit values plus scale bytes",
and of "DeepSeek V4.1 Flash 深度解析", part 4 entry on FP4 in the KV cache,
which keeps the sliding window in FP8):

* FP4 E2M1 (OCP MX v1.0): 1 sign, 2 exponent (bias 1), 1 mantissa bit,
  no inf / NaN.  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
* FP8 E4M3 "fn" (OCP): 1 sign, 4 exponent (bias 7), 3 mantissa bits,
  no inf, NaN = S.1111.111, max 448.
* bfloat16: the top 16 bits of an IEEE binary32.
"""
from __future__ import annotations

import numpy as np


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """u8 [..., n] -> 4-bit codes [..., 2n]; element 2i is the LOW nibble of byte i."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out


def e2m1_decode(code: np.ndarray) -> np.ndarray:
    """4-bit E2M1 codes -> float64.

    sign = bit 3, exponent = bits 2..1, mantissa = bit 0.
    exponent 0 is subnormal: mantissa * 2^(1-1) * 0.5; otherwise
    (1 + mantissa/2) * 2^(exponent-1).
    """
    c = np.asarray(code, dtype=np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m * 0.5) * np.exp2(e - 1.0))
    return np.where(s == 1, -mag, mag).astype(np.float64)


def e4m3_decode(byte: np.ndarray) -> np.ndarray:
    """E4M3 (OCP "fn") bytes -> float64; S.1111.111 decodes to NaN."""
    b = np.asarray(byte, dtype=np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag).astype(np.float64)


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (any 16-bit integer dtype) -> float64."""
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)
