"""Plain fp64 CPU oracle of the CSA2 decode / prefill step.  TEST INFRASTRUCTURE.

Nothing here is tuned: every function is the definition written out with
numpy, one step after another, so it can be checked by eye against the pages.
It shares no code with the HIP library and imports nothing from it.

Pages cited (by title; sections named where used):
  [STRUCT] "DeepSeek-V4.1 模型结构（0）：一张图看懂 DeepSeek-V4.1-Flash" (xhh.club)
  [DEEP]   "DeepSeek V4.1 Flash 深度解析" (daiw.net column index)
  [V4TO41] "从V4到V4.1 Flash：架构的激进进化" (prism.simon-ai.net video summary)

Readings taken where the pages are silent (each is also listed in the design notes):
  R1  score = fp32 entry scale x (bf16 query . E2M1 codes), a plain dot product.
  R2  top-k ties go to the lowest entry index; the output list is ascending, -1 padded.
  R3  pool = the decoder Full layer's top-16,384 under its own score; Reindex re-scores
      only the pool and its ties go to the lowest ENTRY index.
  R4  every selected main entry and every sliding-window row is both key and value;
      one softmax over their union, scale 1/sqrt(512); no sink, bias or RoPE.
  R5  an entry with ratio r covering tokens [j*r, j*r + r - 1] is visible to a query at
      position p once j*r + r - 1 <= p; the window holds positions max(0,p-127)..p.
  R6  sliding-window rows are raw E4M3 (no scale).
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

from .formats import bf16_decode, e2m1_decode, e4m3_decode, unpack_nibbles

D_IDX = 128      # indexer key / query width
D_KV = 512       # main KV width
N_HEADS = 16     # query heads sharing each entry (one KV head)
SWA_W = 128      # sliding-window length
TOPK = 512       # entries each Full / Reindex layer selects
POOL = 16384     # decoder candidate pool (the pages' "about 16,00[0]" positions)
SCALE_GROUP = 16  # main-KV values per E4M3 scale byte

# Layer modes of the 40-layer backbone ([STRUCT], Q&A on how the 40 layers are laid out):
# layers 0-1 sliding window only; Full at 2, 8, 14, 20; Reindex at 24, 28, 32, 36;
# every other layer Reuse.  Layers 0-19 form the encoder, 20-39 the decoder.
N_LAYERS = 40
SWA_ONLY_LAYERS = (0, 1)
FULL_LAYERS = (2, 8, 14, 20)
REINDEX_LAYERS = (24, 28, 32, 36)
FIRST_DECODER_LAYER = 20


# ----------------------------------------------------------------------------
# Byte accounting ([STRUCT], Q&A on how the 890-byte figure is derived, and the
# Q&A on the compression result at a 1M context).
# ----------------------------------------------------------------------------
def index_entry_bytes() -> int:
    """128 values of 4 bits plus one 4-byte scale."""
    return D_IDX * 4 // 8 + 4


def main_entry_bytes() -> int:
    """512 values of 4 bits plus one E4M3 scale byte per 16 values (32 bytes)."""
    return D_KV * 4 // 8 + D_KV // SCALE_GROUP


def layer_mode(layer: int) -> str:
    if layer in SWA_ONLY_LAYERS:
        return "swa"
    if layer in FULL_LAYERS:
        return "full"
    if layer in REINDEX_LAYERS:
        return "reindex"
    return "reuse"


def reuse_source(layer: int) -> int:
    """Layer whose index list a Reuse layer attends over: the most recent Full or
    Reindex layer at or below it ([V4TO41], section on the CSA2 architecture:
    a Reuse layer takes the earlier layer's KV and top-k indices)."""
    for l in range(layer, -1, -1):
        if layer_mode(l) in ("full", "reindex"):
            return l
    raise ValueError(f"layer {layer} has no Full/Reindex layer below it")


def entries_per_token(enc_ratio: int = 2, dec_ratio: int = 1) -> float:
    """Global entries stored per context token: one pool per Full layer, each
    compressed at its ratio ([V4TO41], encoder section: 1:2 in the encoder;
    decoder section: no token compression in the decoder)."""
    n = 0.0
    for l in FULL_LAYERS:
        n += 1.0 / (dec_ratio if l >= FIRST_DECODER_LAYER else enc_ratio)
    return n


def global_kv_bytes_per_token() -> float:
    return (index_entry_bytes() + main_entry_bytes()) * entries_per_token()


def global_kv_bytes(ctx_tokens: int) -> float:
    return global_kv_bytes_per_token() * ctx_tokens


# ----------------------------------------------------------------------------
# a1 / a3: indexer score (reading R1)
# ----------------------------------------------------------------------------
def dequant_index_keys(codes: np.ndarray) -> np.ndarray:
    """u8 [n, 64] -> unscaled E2M1 values fp64 [n, 128]."""
    return e2m1_decode(unpack_nibbles(codes))


def index_dot_is_exact(q_idx_bits: np.ndarray) -> bool:
    """True when q . v is exact in fp64 for every possible E2M1 key v.

    Every product q_d * v_d is a multiple of u = min_d ulp(q_d) * 0.5 (E2M1 values
    are multiples of 0.5), so each partial sum is an integer multiple of u.  If
    sum_d |q_d| * 6 < 2^53 * u, every partial sum fits in 53 bits and the fp64 sum
    is exact in any order."""
    q = bf16_decode(q_idx_bits)
    nz = np.abs(q[q != 0])
    if nz.size == 0:
        return True
    e = np.floor(np.log2(nz))
    ulp = np.exp2(np.maximum(e, -126.0) - 7.0)
    u = ulp.min() * 0.5
    return bool(nz.sum() * 6.0 < 2.0 ** 53 * u)


def index_scores(q_idx_bits: np.ndarray, codes: np.ndarray, scale: np.ndarray,
                 chunk: int = 1 << 16) -> np.ndarray:
    """s_j = scale_j * sum_d q_d * e2m1(c_jd), in fp64.

    The dot is exact (see index_dot_is_exact); the product with the fp32 scale is
    rounded once to fp64."""
    q = bf16_decode(q_idx_bits).reshape(D_IDX)
    n = codes.shape[0]
    out = np.empty(n, dtype=np.float64)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        dot = dequant_index_keys(codes[s:e]) @ q
        out[s:e] = np.asarray(scale[s:e], dtype=np.float32).astype(np.float64) * dot
    return out


# ----------------------------------------------------------------------------
# a2: top-k selection (reading R2)
# ----------------------------------------------------------------------------
def topk(scores: np.ndarray, k: int, n_valid: Optional[int] = None) -> np.ndarray:
    """Indices of the k largest scores, ties to the lower index, listed ascending,
    -1 padded when fewer than k are visible.  A full sort: brute force."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0] if n_valid is None else int(n_valid)
    s = s[:n]
    order = np.lexsort((np.arange(n), -s))  # primary key -s (score descending), then index
    take = np.sort(order[: min(k, n)])
    out = np.full(k, -1, dtype=np.int32)
    out[: take.size] = take
    return out


def full_layer(q_idx_bits, idx_codes, idx_scale, n_valid: int,
               pool_size: Optional[int] = POOL, k: int = TOPK):
    """Full mode: score every visible entry, take the pool (decoder only) and the
    layer's own top-k ([STRUCT], commentary on the four layer modes; [V4TO41],
    decoder section on the hierarchical coarse indexer: the first layer scans
    everything and builds a pool of about 16K positions)."""
    s = index_scores(q_idx_bits, idx_codes[:n_valid], idx_scale[:n_valid])
    pool = topk(s, pool_size) if pool_size else None
    own = topk(s, k)
    return s, pool, own


def reindex_layer(q_idx_bits, idx_codes, idx_scale, pool: np.ndarray, k: int = TOPK):
    """Reindex mode: re-score only the pool's entries with the layer's own indexer
    query and take the top-k of those ([STRUCT], commentary on the four layer
    modes; [V4TO41], CSA2 architecture section).  Ties go to the lower entry id.
    Returns (entry ids ascending, -1 padded; the scores of the pool entries)."""
    ids = np.asarray(pool)[np.asarray(pool) >= 0].astype(np.int64)
    s = index_scores(q_idx_bits, idx_codes[ids], idx_scale[ids])
    order = np.lexsort((ids, -s))
    take = np.sort(ids[order[: min(k, ids.size)]])
    out = np.full(k, -1, dtype=np.int32)
    out[: take.size] = take
    return out, s


def reuse_layer(indices: np.ndarray) -> np.ndarray:
    """Reuse mode: no indexer; the layer attends over the source layer's list as is
    ([V4TO41], CSA2 architecture section)."""
    return np.array(indices, copy=True)


# ----------------------------------------------------------------------------
# a5 / a6: gather-dequant and attention (readings R4, R6)
# ----------------------------------------------------------------------------
def dequant_main(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """u8 [m, 256] codes and u8 [m, 32] E4M3 scales -> fp64 [m, 512]:
    value[e] = e2m1(code[e]) * e4m3(scale[e // 16])."""
    v = e2m1_decode(unpack_nibbles(codes))
    s = e4m3_decode(scale)
    return v * np.repeat(s, SCALE_GROUP, axis=-1)


def dequant_swa(rows: np.ndarray) -> np.ndarray:
    """u8 [w, 512] E4M3 -> fp64 [w, 512]."""
    return e4m3_decode(rows)


def attention(q_bits: np.ndarray, values: np.ndarray, softmax_scale: float) -> np.ndarray:
    """out_h = sum_j softmax_j(z_h) v_j with z_hj = (q_h . v_j) * scale; every row of
    ``values`` is both key and value.  Empty set -> zeros."""
    q = bf16_decode(q_bits).reshape(N_HEADS, D_KV)
    if values.shape[0] == 0:
        return np.zeros((N_HEADS, D_KV), dtype=np.float64)
    z = (q @ values.T) * softmax_scale
    m = z.max(axis=1, keepdims=True)
    w = np.exp(z - m)
    return (w @ values) / w.sum(axis=1, keepdims=True)


def decode_attention(q_bits, kv_codes, kv_scale, seq_base: int, idx: np.ndarray,
                     swa_rows: np.ndarray, swa_len: int,
                     softmax_scale: float = 1.0 / math.sqrt(D_KV)) -> np.ndarray:
    """Sparse attention of one query over its selected entries (idx, -1 skipped)
    merged in one softmax with the first ``swa_len`` window rows ([V4TO41],
    section on global KV sharing with separate per-layer sliding windows)."""
    sel = np.asarray(idx)
    sel = sel[sel >= 0].astype(np.int64) + int(seq_base)
    parts = [dequant_main(kv_codes[sel], kv_scale[sel]),
             dequant_swa(np.asarray(swa_rows)[: int(swa_len)])]
    return attention(q_bits, np.concatenate(parts, axis=0), softmax_scale)


# ----------------------------------------------------------------------------
# a7 / a8: prefill chunk (reading R5)
# ----------------------------------------------------------------------------
def visible_entries(pos: int, ratio: int, n_entries: int) -> int:
    """Entries whose last token is at or before ``pos``: j*ratio + ratio - 1 <= pos."""
    return max(0, min(int(n_entries), (int(pos) + 1) // int(ratio)))


def prefill_chunk(q_idx_bits, q_bits, idx_codes, idx_scale, kv_codes, kv_scale,
                  n_entries: int, ratio: int, pos0: int, k: int, swa_rows,
                  softmax_scale: float = 1.0 / math.sqrt(D_KV),
                  rows: Optional[Sequence[int]] = None):
    """Each query t (position pos0 + t) scores its causally visible entries, takes its
    own top-k and attends over them plus the window positions max(0,p-127)..p.
    ``swa_rows[r]`` holds position pos0 - 127 + r.

    The chunk runs one Full layer of the encoder over the prompt ([STRUCT], content
    summary and the Q&A on prefill: prompt tokens pass only the encoder layers)."""
    T = q_idx_bits.shape[0]
    rows = range(T) if rows is None else rows
    keys = dequant_index_keys(idx_codes[:n_entries])          # decoded once, reused per row
    kscale = np.asarray(idx_scale[:n_entries], dtype=np.float32).astype(np.float64)
    idx_out, out = {}, {}
    for t in rows:
        p = pos0 + t
        n_t = visible_entries(p, ratio, n_entries)
        q = bf16_decode(q_idx_bits[t])
        s = kscale[:n_t] * (keys[:n_t] @ q)
        sel = topk(s, k)
        lo = max(0, p - (SWA_W - 1))
        r0 = lo - (pos0 - (SWA_W - 1))
        r1 = p - (pos0 - (SWA_W - 1)) + 1
        win = np.asarray(swa_rows)[r0:r1]
        idx_out[t] = sel
        out[t] = decode_attention(q_bits[t], kv_codes, kv_scale, 0, sel, win, win.shape[0],
                                  softmax_scale)
    return idx_out, out


# ----------------------------------------------------------------------------
# Decode compositions
# ----------------------------------------------------------------------------
def decode_step_long(q_idx_full, q_idx_reindex, q_bits, idx_codes, idx_scale, kv_codes,
                     kv_scale, seq_base: int, n_valid: int, swa_rows, swa_len: int,
                     pool_size: int = POOL, k: int = TOPK):
    """Decoder step at long context: Full scan -> pool -> one Reindex top-k ->
    sparse attention with the window.  Returns (pool, idx, out)."""
    b = int(seq_base)
    _, pool, _ = full_layer(q_idx_full, idx_codes[b:b + n_valid], idx_scale[b:b + n_valid],
                            n_valid, pool_size, k)
    idx, _ = reindex_layer(q_idx_reindex, idx_codes[b:b + n_valid], idx_scale[b:b + n_valid],
                           pool, k)
    out = decode_attention(q_bits, kv_codes, kv_scale, b, idx, swa_rows, swa_len)
    return pool, idx, out


def decoder_chain(q_idx_layers: Dict[int, np.ndarray], q_layers: Dict[int, np.ndarray],
                  swa_layers: Dict[int, np.ndarray], swa_len: int,
                  idx_codes, idx_scale, kv_codes, kv_scale, seq_base: int, n_valid: int,
                  pool_size: int = POOL, k: int = TOPK,
                  first: int = FIRST_DECODER_LAYER, last: int = N_LAYERS - 1):
    """Layers first..last of one sequence: Full builds the pool and its own top-k,
    Reindex layers re-pick inside the pool, Reuse layers attend over the list of
    their source layer.  Returns {layer: (idx, out)} and the pool."""
    b = int(seq_base)
    codes, scale = idx_codes[b:b + n_valid], idx_scale[b:b + n_valid]
    lists: Dict[int, np.ndarray] = {}
    result = {}
    pool = None
    for layer in range(first, last + 1):
        mode = layer_mode(layer)
        if mode == "full":
            _, pool, lists[layer] = full_layer(q_idx_layers[layer], codes, scale, n_valid,
                                               pool_size, k)
        elif mode == "reindex":
            lists[layer], _ = reindex_layer(q_idx_layers[layer], codes, scale, pool, k)
        elif mode == "reuse":
            lists[layer] = reuse_layer(lists[reuse_source(layer)])
        else:
            lists[layer] = np.full(k, -1, dtype=np.int32)
        out = decode_attention(q_layers[layer], kv_codes, kv_scale, b, lists[layer],
                               swa_layers[layer], swa_len)
        result[layer] = (lists[layer], out)
    return result, pool
