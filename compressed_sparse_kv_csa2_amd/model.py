"""One decode step of the 40-layer CSA2 backbone, sequenced through the C ABI.

Sequencing only: every step runs in the library's kernels (csa2_index_topk,
csa2_select_chain, csa2_replay_select, csa2_sparse_attn_decode, csa2_sparse_attn_prefill); this module holds workspaces and output
buffers and issues the calls in layer order on one stream.

Layer layout ("DeepSeek-V4.1 模型结构（0）：一张图看懂 DeepSeek-V4.1-Flash", Q&A on how the
40 layers are laid out, and commentary on the four layer modes; "从V4到V4.1 Flash：架构的
激进进化", CSA2 architecture, encoder and decoder sections):
  * layers 0-1 attend their sliding window only;
  * Full at 2, 8 and 14 (encoder: each scans its own 1:2 pool and takes its top-512) and at
    20 (decoder: scans the ratio-1 pool, keeps the top-16,384 as the candidate pool and its
    own top-512 inside it);
  * Reindex at 24, 28, 32, 36: the layer's own indexer query re-scores the pool only;
  * every other layer is Reuse: the list of the most recent Full/Reindex layer at or below
    it;
  * every layer attends with its own 16 x 512 query over its list plus its own 128-row
    window.
Each Reindex layer's query arrives at its own layer (it depends on the layers before it in
a real decoder), so the Reindex selections run per layer: csa2_index_topk over the pool
(for pools of up to 16,384 one launch scores the pool and the last workgroup of each row
selects).
"""
from __future__ import annotations

import torch

from . import (attn_workspace, csa2_index_topk, csa2_replay_select, csa2_select_chain,
               csa2_sparse_attn_decode, csa2_sparse_attn_prefill, index_topk_workspace,
               replay_select_workspace, select_chain_workspace)

N_LAYERS = 40
WINDOW_ONLY = (0, 1)
ENCODER_FULL = (2, 8, 14)
DECODER_FULL = 20
REINDEX = (24, 28, 32, 36)
SELECTING = ENCODER_FULL + (DECODER_FULL,) + REINDEX


def list_source(layer: int) -> int:
    """The layer whose selection `layer` attends over (itself for Full/Reindex layers)."""
    return max(l for l in SELECTING if l <= layer)


class DecodePass:
    """Buffers for one 40-layer decode step of `batch` sequences.

    enc_entries / dec_entries: entries per sequence in each encoder pool / the decoder pool.
    After step(): lists[l] (int32 [batch, k]) for every selecting layer, pool (int32
    [batch, pool]) and out[l] (f32 [batch, 16, 512]) for every layer."""

    def __init__(self, batch: int, enc_entries: int, dec_entries: int, pool: int = 16384,
                 k: int = 512, device="cuda"):
        self.B, self.n_enc, self.n_dec, self.P, self.K = batch, enc_entries, dec_entries, pool, k
        dev = torch.device(device)
        self.enc_ws = index_topk_workspace(batch, enc_entries, k, device=dev)
        self.dec_ws = select_chain_workspace(batch, dec_entries, pool, device=dev)
        self.re_ws = index_topk_workspace(batch, pool, k, device=dev)  # Reindex: the pool re-scored
        self.attn_ws = attn_workspace(batch, k, device=dev)
        self.pool = torch.empty((batch, pool), dtype=torch.int32, device=dev)
        self.pool_valid = torch.full((batch,), pool, dtype=torch.int32, device=dev)
        self.lists = {l: torch.empty((batch, k), dtype=torch.int32, device=dev) for l in SELECTING}
        self.out = torch.empty((N_LAYERS, batch, 16, 512), dtype=torch.float32, device=dev)
        self._calls, self._calls_key = None, None  # the prepared calls of the last inputs

    def workspaces(self):
        """The selection workspaces whose status block (csa2_workspace_status) reports errors."""
        return [self.enc_ws, self.dec_ws, self.re_ws]

    def step(self, enc_caches, dec_cache, q_idx, q, swa, swa_len, stream=None, marks=None):
        """enc_caches: three entry caches (layers 2, 8, 14); dec_cache: the decoder's.
        q_idx: {selecting layer: bf16 [batch, 128]}; q: bf16 [40, batch, 16, 512];
        swa: E4M3 [40, batch, 128, 512]; swa_len: int32 [batch].  marks (optional): four
        events recorded before layer 0, around the decoder's Full selection and at the end.

        The 40 layers' calls are checked and marshalled once and issued again on later steps
        whose inputs are the same buffers (addresses, shapes, strides, dtypes) on the same
        stream: the host's cost per call is then the C call alone."""
        if stream is None:
            stream = torch.cuda.current_stream()
        key = self._key(enc_caches, dec_cache, q_idx, q, swa, swa_len, stream)
        if key != self._calls_key:
            self._calls = self._prepare(enc_caches, dec_cache, q_idx, q, swa, swa_len, stream)
            self._calls_key = key
        if marks is not None:
            marks[0].record(stream)
        for l, (select, attend) in enumerate(self._calls):
            if l == DECODER_FULL and marks is not None:
                marks[1].record(stream)
            if select is not None:
                select()
            if l == DECODER_FULL and marks is not None:
                marks[2].record(stream)
            attend()
        if marks is not None:
            marks[3].record(stream)

    @staticmethod
    def _key(enc_caches, dec_cache, q_idx, q, swa, swa_len, stream):
        def t(x):
            return (x.data_ptr(), tuple(x.shape), x.stride(), x.dtype)

        def cache(c):
            return (t(c.idx_codes), t(c.idx_scale), t(c.seq_base), t(c.n_entries), t(c.kv_codes),
                    t(c.kv_scale))

        return (stream.cuda_stream, tuple(cache(c) for c in enc_caches), cache(dec_cache),
                tuple(t(q_idx[l]) for l in SELECTING), t(q), t(swa), t(swa_len))

    def _prepare(self, enc_caches, dec_cache, q_idx, q, swa, swa_len, stream):
        """(selection or None, attention) per layer, checked and marshalled."""
        calls = []
        for l in range(N_LAYERS):
            select = None
            if l in ENCODER_FULL:
                c = enc_caches[ENCODER_FULL.index(l)]
                select = csa2_index_topk(q_idx[l], c.idx_codes, c.idx_scale, c.seq_base, c.n_entries,
                                         self.K, self.lists[l], self.enc_ws, self.n_enc, stream=stream,
                                         prepare=True)
            elif l == DECODER_FULL:
                c = dec_cache
                select = csa2_select_chain(q_idx[l], c.idx_codes, c.idx_scale, c.seq_base, c.n_entries,
                                           self.n_dec, self.pool, self.dec_ws, k=self.K,
                                           own_out=self.lists[l], stream=stream, prepare=True)
            elif l in REINDEX:
                c = dec_cache
                select = csa2_index_topk(q_idx[l], c.idx_codes, c.idx_scale, c.seq_base, self.pool_valid,
                                         self.K, self.lists[l], self.re_ws, self.P, cand=self.pool,
                                         stream=stream, prepare=True)
            if l in WINDOW_ONLY:
                c, idx = dec_cache, None
            else:
                src = list_source(l)
                c = dec_cache if src >= DECODER_FULL else enc_caches[ENCODER_FULL.index(src)]
                idx = self.lists[src]
            attend = csa2_sparse_attn_decode(q[l], c.kv_codes, c.kv_scale, c.seq_base, idx, swa[l],
                                             swa_len, self.out[l], self.attn_ws, stream=stream,
                                             prepare=True)
            calls.append((select, attend))
        return calls


class ReplayChunk:
    """The decoder's bounded replay: T consecutive tokens of one sequence (positions pos0 ..
    pos0 + T - 1) through the decoder's 20 layers ("DeepSeek-V4.1 模型结构（0）：一张图看懂
    DeepSeek-V4.1-Flash", content summary and Q&A on prefill: on eviction or restore only the
    last 128 tokens of the decoder are replayed; "从V4到V4.1 Flash：架构的激进进化", decoder
    section).  The decoder's global KV has ratio 1, so entry j is token j and query t sees
    entries 0 .. pos0 + t.  Per query, as in decode: the Full layer (20) scores every visible
    entry, keeps its top-16,384 as the query's pool and its own top-512 inside it
    (csa2_replay_select: one MFMA contraction reads the keys once for all T queries, and the
    library derives each query's visible entries from pos0); each Reindex layer re-scores
    that query's pool; every layer attends over its list and its own causal window.

    After step(): pool (int32 [T, pool]), lists[l] (int32 [T, k]) for 20, 24, 28, 32, 36 and
    out[l - 20] (f32 [T, 16, 512]) for layers 20..39."""

    def __init__(self, T: int, n_entries: int, pos0: int, pool: int = 16384, k: int = 512,
                 device="cuda"):
        self.T, self.n, self.pos0, self.P, self.K = T, n_entries, pos0, pool, k
        dev = torch.device(device)
        self.sel_ws = replay_select_workspace(T, n_entries, pool, device=dev)
        self.attn_ws = attn_workspace(T, k, device=dev)
        self.re_ws = index_topk_workspace(T, pool, k, device=dev)  # Reindex: the pool re-scored
        self.seq_base = torch.zeros((T,), dtype=torch.int64, device=dev)
        self.pool = torch.empty((T, pool), dtype=torch.int32, device=dev)
        self.pool_valid = torch.empty((T,), dtype=torch.int32, device=dev)  # written by the selection
        self.lists = {l: torch.empty((T, k), dtype=torch.int32, device=dev)
                      for l in (DECODER_FULL,) + REINDEX}
        self.out = torch.empty((N_LAYERS - DECODER_FULL, T, 16, 512), dtype=torch.float32, device=dev)

    def workspaces(self):
        """The selection workspaces whose status block (csa2_workspace_status) reports errors."""
        return [self.sel_ws, self.re_ws]

    def step(self, cache, q_idx, q, swa, stream=None, marks=None):
        """cache: the sequence's decoder entries (planes from entry 0); q_idx: {20, 24, 28,
        32, 36: bf16 [T, 128]}; q: bf16 [20, T, 16, 512] (layers 20..39); swa: E4M3
        [20, T + 127, 512] (row r = position pos0 - 127 + r).  marks (optional): three events,
        before the Full selection, after it, at the end."""
        if marks is not None:
            marks[0].record(stream)
        csa2_replay_select(q_idx[DECODER_FULL], cache.idx_codes, cache.idx_scale, self.n, 1, self.pos0,
                           self.pool, self.sel_ws, k=self.K, own_out=self.lists[DECODER_FULL],
                           pool_n_out=self.pool_valid, stream=stream)
        if marks is not None:
            marks[1].record(stream)
        for l in range(DECODER_FULL, N_LAYERS):
            if l in REINDEX:
                csa2_index_topk(q_idx[l], cache.idx_codes, cache.idx_scale, self.seq_base, self.pool_valid,
                                self.K, self.lists[l], self.re_ws, self.P, cand=self.pool, stream=stream)
            csa2_sparse_attn_prefill(q[l - DECODER_FULL], cache.kv_codes, cache.kv_scale,
                                     self.lists[list_source(l)], swa[l - DECODER_FULL], self.pos0,
                                     self.out[l - DECODER_FULL], self.attn_ws, stream=stream)
        if marks is not None:
            marks[2].record(stream)
