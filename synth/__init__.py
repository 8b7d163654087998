"""Seeded synthetic inputs for the CSA2 decode and prefill path.

This module only draws and packs inputs.  It holds no scoring, selection,
dequantisation or attention arithmetic, so the CPU oracle (``oracle/``) and
the HIP library (``compressed_sparse_kv_csa2_amd``) can both be fed from it
without sharing any of the method's code.

Recipe (every value is N(0,1) before it is stored):

* indexer keys: 128 values per entry, one fp32 scale ``amax/6`` per entry,
  each value rounded to nearest-even on the FP4 E2M1 grid after division by
  the scale (saturating at 6).  64 code bytes + 4 scale bytes = 68 B.
* main KV: 512 values per entry, one E4M3 scale per 16 values
  (``e4m3(amax/6)``, round-to-nearest-even), E2M1 codes as above.
  256 code bytes + 32 scale bytes = 288 B.
* sliding window: raw E4M3 of N(0,1) values, 512 per row.
* indexer queries (128-d) and attention queries (16 x 512) in bf16.

Nibble order: element ``2i`` is the low nibble of byte ``i``.

Streams are ``torch.Generator`` objects seeded from ``(seed, field)``, so the
same seed gives the same bytes on the same device kind.  Large workloads are
drawn on the GPU (fast); small test cases can be drawn on the CPU.

Byte formats follow "DeepSeek-V4.1 模型结构（0）：一张图看懂 DeepSeek-V4.1-Flash",
Q&A on how the 890-byte global KV figure is derived (288 B main entry,
68 B indexer entry), and "DeepSeek V4.1 Flash 深度解析", part 4 entry on FP4
moving into the KV cache (main KV in 4 bit, in a format unlike the indexer's;
sliding window kept in FP8).  The exact codes (E2M1 / E4M3, OCP MX) are a
reading of those passages, not stated on the pages.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np
import torch

D_IDX = 128
D_KV = 512
N_HEADS = 16
SWA_W = 128

# Field ids for independent random streams.
F_IDX_KEYS, F_KV, F_QIDX, F_Q, F_SWA = 0, 1, 2, 3, 4

# Magnitudes of the E2M1 grid, indexed by the 3-bit magnitude code, used only
# to ENCODE inputs; decoding lives separately in the oracle and in the kernels.
_E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
_E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _gen(device: torch.device, seed: int, field: int, sub: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + field * 10_007 + sub) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def _randn(shape, g: torch.Generator, device) -> torch.Tensor:
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def e2m1_encode(y: torch.Tensor) -> torch.Tensor:
    """Round f32 values to nearest-even E2M1 codes (uint8 0..15), saturating at +-6."""
    mag = y.abs()
    mids = torch.tensor(_E2M1_MIDPOINTS, device=y.device, dtype=torch.float32)
    code = torch.bucketize(mag, mids, right=False)  # number of midpoints strictly below mag
    # bucketize(right=False) returns i with mids[i-1] < mag <= mids[i]; a value equal to a
    # midpoint lands on the lower code i.  Ties go to the even code.
    safe = code.clamp(max=len(_E2M1_MIDPOINTS) - 1)
    at_mid = (code < len(_E2M1_MIDPOINTS)) & (mag == mids[safe])
    code = torch.where(at_mid & (code % 2 == 1), code + 1, code)
    code = code.to(torch.uint8)
    sign = torch.signbit(y).to(torch.uint8)
    return code | (sign << 3)


def e2m1_grid_value(code: torch.Tensor) -> torch.Tensor:
    """Encoder-side value of a code (for generator bookkeeping and pins)."""
    grid = torch.tensor(_E2M1_GRID, device=code.device, dtype=torch.float32)
    v = grid[(code & 7).long()]
    return torch.where((code & 8) != 0, -v, v)


def pack_nibbles(codes: torch.Tensor) -> torch.Tensor:
    """[..., 2n] codes -> [..., n] bytes, element 2i in the low nibble."""
    lo = codes[..., 0::2]
    hi = codes[..., 1::2]
    return (lo | (hi << 4)).contiguous()


def quantize_index_keys(x: torch.Tensor):
    """x f32 [n, 128] -> (codes u8 [n, 64], scale f32 [n], values f32 [n, 128])."""
    amax = x.abs().amax(dim=-1)
    scale = amax / 6.0
    scale = torch.where(scale > 0, scale, torch.ones_like(scale))
    codes = e2m1_encode(x / scale[:, None])
    values = e2m1_grid_value(codes) * scale[:, None]
    return pack_nibbles(codes), scale.contiguous(), values


def quantize_main_kv(x: torch.Tensor):
    """x f32 [n, 512] -> (codes u8 [n, 256], scale u8 [n, 32] E4M3, values f32 [n, 512])."""
    n = x.shape[0]
    g = x.view(n, D_KV // 16, 16)
    amax = g.abs().amax(dim=-1)
    s8 = (amax / 6.0).to(torch.float8_e4m3fn)
    sbits = s8.view(torch.uint8)
    sbits = torch.where(sbits == 0, torch.ones_like(sbits), sbits)  # never a zero scale
    s = sbits.view(torch.float8_e4m3fn).to(torch.float32)
    codes = e2m1_encode(g / s[..., None]).view(n, D_KV)
    values = (e2m1_grid_value(codes).view(n, D_KV // 16, 16) * s[..., None]).view(n, D_KV)
    return pack_nibbles(codes), sbits.contiguous(), values


def e4m3_bytes(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """f32 -> bf16 (RNE) bit patterns as int16 storage (reinterpret as uint16 on the host)."""
    return x.to(torch.bfloat16).view(torch.int16)


@dataclasses.dataclass
class EntryCache:
    """Packed global-KV entries for several sequences laid out back to back."""
    idx_codes: torch.Tensor   # u8 [n_total, 64]
    idx_scale: torch.Tensor   # f32 [n_total]
    kv_codes: torch.Tensor    # u8 [n_total, 256]
    kv_scale: torch.Tensor    # u8 [n_total, 32]
    seq_base: torch.Tensor    # int64 [B]  first entry of each sequence
    n_entries: torch.Tensor   # int32 [B]

    def to(self, device) -> "EntryCache":
        return EntryCache(*(getattr(self, f.name).to(device) for f in dataclasses.fields(self)))


def make_entries(counts: List[int], seed: int, device="cpu", field_base: int = 0,
                 chunk: int = 1 << 16, keep_values: bool = False):
    """Draw and pack ``sum(counts)`` entries (sequence b holds ``counts[b]``).

    Returns an EntryCache and, if ``keep_values``, the dequantised f32 values
    the generator intended ([n, 128] and [n, 512]) for use as pins.
    """
    device = torch.device(device)
    total = int(sum(counts))
    idx_codes = torch.empty((total, D_IDX // 2), dtype=torch.uint8, device=device)
    idx_scale = torch.empty((total,), dtype=torch.float32, device=device)
    kv_codes = torch.empty((total, D_KV // 2), dtype=torch.uint8, device=device)
    kv_scale = torch.empty((total, D_KV // 16), dtype=torch.uint8, device=device)
    vals_idx = torch.empty((total, D_IDX), dtype=torch.float32, device=device) if keep_values else None
    vals_kv = torch.empty((total, D_KV), dtype=torch.float32, device=device) if keep_values else None
    g_idx = _gen(device, seed, F_IDX_KEYS + field_base)
    g_kv = _gen(device, seed, F_KV + field_base)
    for s in range(0, total, chunk):
        e = min(total, s + chunk)
        c, sc, v = quantize_index_keys(_randn((e - s, D_IDX), g_idx, device))
        idx_codes[s:e], idx_scale[s:e] = c, sc
        if keep_values:
            vals_idx[s:e] = v
        c, sc, v = quantize_main_kv(_randn((e - s, D_KV), g_kv, device))
        kv_codes[s:e], kv_scale[s:e] = c, sc
        if keep_values:
            vals_kv[s:e] = v
    base = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int64)
    cache = EntryCache(idx_codes, idx_scale, kv_codes, kv_scale,
                       torch.tensor(base, dtype=torch.int64, device=device),
                       torch.tensor(counts, dtype=torch.int32, device=device))
    if keep_values:
        return cache, vals_idx, vals_kv
    return cache


def make_index_queries(B: int, seed: int, device="cpu", sub: int = 0) -> torch.Tensor:
    """bf16 bits (int16 storage) [B, 128]."""
    device = torch.device(device)
    return bf16_bits(_randn((B, D_IDX), _gen(device, seed, F_QIDX, sub), device))


def make_queries(B: int, seed: int, device="cpu", sub: int = 0) -> torch.Tensor:
    """bf16 bits (int16 storage) [B, 16, 512]."""
    device = torch.device(device)
    return bf16_bits(_randn((B, N_HEADS, D_KV), _gen(device, seed, F_Q, sub), device))


def make_swa(B: int, rows: int, seed: int, device="cpu", sub: int = 0) -> torch.Tensor:
    """E4M3 bytes [B, rows, 512]."""
    device = torch.device(device)
    return e4m3_bytes(_randn((B, rows, D_KV), _gen(device, seed, F_SWA, sub), device))


F_APPEND_IDX, F_APPEND_KV, F_APPEND_SWA = 5, 6, 7


def make_append_vectors(n: int, seed: int, device="cpu"):
    """New global-KV vectors before quantisation: bf16 bits (int16 storage) [n, 128] and
    [n, 512], N(0,1) times a per-row magnitude drawn log-uniformly from 2^-8 .. 2^8 (the
    magnitude only spreads the scales; both sides read the same bits)."""
    device = torch.device(device)
    g_i, g_k = _gen(device, seed, F_APPEND_IDX), _gen(device, seed, F_APPEND_KV)
    mi = torch.exp2(torch.rand((n, 1), generator=g_i, device=device) * 16 - 8)
    mk = torch.exp2(torch.rand((n, 1), generator=g_k, device=device) * 16 - 8)
    return (bf16_bits(_randn((n, D_IDX), g_i, device) * mi),
            bf16_bits(_randn((n, D_KV), g_k, device) * mk))


def make_window_rows(B: int, seed: int, device="cpu") -> torch.Tensor:
    """New window rows before quantisation: bf16 bits (int16 storage) [B, 512], N(0,1)."""
    device = torch.device(device)
    return bf16_bits(_randn((B, D_KV), _gen(device, seed, F_APPEND_SWA), device))


# ----------------------------------------------------------------------------
# The five workloads (sizes as the path's configurations state them).
# ----------------------------------------------------------------------------
CONFIGS: Dict[str, dict] = {
    # 1 query, ctx 4096 compressed 1:2 -> 2048 entries, Full, top-512.
    "c1_tiny_full": dict(seed=0, B=1, ctx=4096, ratio=2, k=512, pool=None),
    # 32 sequences x 65,536 ctx (1:2 -> 32,768 entries), Full, top-512.
    "c2_batched_full": dict(seed=1, B=32, ctx=65536, ratio=2, k=512, pool=None),
    # 16 sequences x 131,072 ctx at ratio 1; 1 Full (pool 16,384 + own top-512),
    # 4 Reindex, 15 Reuse.
    "c3_decoder_chain": dict(seed=2, B=16, ctx=131072, ratio=1, k=512, pool=16384,
                             n_reindex=4, n_reuse=15),
    # 4 sequences at 2^20 ctx; decoder pool at ratio 1 (1,048,576 entries), three
    # encoder pools at 1:2 (524,288 entries each); Full scan -> pool 16,384 ->
    # Reindex top-512 -> attention.
    "c4_long_decode": dict(seed=3, B=4, ctx=1 << 20, ratio=1, k=512, pool=16384,
                           enc_pools=3, enc_ratio=2),
    # Prefill chunk: 4,096 queries at the tail of a 262,144-token context, 1:2.
    "c5_prefill": dict(seed=4, T=4096, ctx=262144, ratio=2, k=512),
}


def entries_for(ctx: int, ratio: int) -> int:
    """Number of compressed entries a context of ``ctx`` tokens yields at ``ratio``."""
    return ctx // ratio
