"""GPU parity of the decoder's bounded replay chunk (compressed_sparse_kv_csa2_amd.model.
ReplayChunk) and of csa2_sparse_attn_prefill against the oracle: per query, the Full
layer's pool of 16,384 and its own top-512 over the causally visible entries (ratio 1),
the four Reindex layers' top-512 inside that query's pool (staged on the GPU's pool), and
every decoder layer's attention over its list and causal window (staged on the GPU's
lists).  Cases: the tail of a 24,000-entry sequence (the pool is a real selection) and the
start of a sequence (fewer visible entries than the pool and than k)."""
import math
import sys

import numpy as np
import pytest
import torch

import compressed_sparse_kv_csa2_amd as csa2
from compressed_sparse_kv_csa2_amd import model
import oracle
import synth
from _util import ATTN_TOL, assert_ws_ok, attn_rel_err, check_topk

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCALE = 1.0 / math.sqrt(512)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def h(t):
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


@pytest.mark.parametrize("n,T,pos0,rows", [
    (24000, 100, 23800, (0, 41, 99)),
    (5000, 128, 0, (0, 1, 100, 127)),
])
def test_replay_chunk(n, T, pos0, rows):
    log(f"replay n={n} T={T} pos0={pos0}")
    seed = 11
    cache = synth.make_entries([n], seed=seed, device=DEV)
    q_idx = {l: synth.make_index_queries(T, seed, device=DEV, sub=l) for l in (20,) + model.REINDEX}
    q = torch.stack([synth.make_queries(T, seed, device=DEV, sub=l) for l in range(20, 40)]).contiguous()
    swa = torch.stack([synth.make_swa(1, T + 127, seed, device=DEV, sub=l)[0] for l in range(20, 40)]).contiguous()
    run = model.ReplayChunk(T, n, pos0, device=DEV)
    run.step(cache, q_idx, q, swa)
    torch.cuda.synchronize()
    assert_ws_ok(*run.workspaces())
    codes, scale = h(cache.idx_codes), h(cache.idx_scale)
    kc, ks = h(cache.kv_codes), h(cache.kv_scale)
    pool = h(run.pool)
    lists = {l: h(v) for l, v in run.lists.items()}
    out, qq, sw = h(run.out), h(q), h(swa)
    for t in range(T):
        vis = min(pos0 + t + 1, n)
        s = oracle.index_scores(h(q_idx[20])[t], codes[:vis], scale[:vis])
        check_topk(pool[t], s, 16384, label=f"pool row {t}")
        p = pool[t][pool[t] >= 0]
        check_topk(lists[20][t], s[p], 512, ids=p, label=f"own row {t}")
        if t in rows:
            for l in model.REINDEX:
                _, r = oracle.reindex_layer(h(q_idx[l])[t], codes, scale, p)
                check_topk(lists[l][t], r, 512, ids=p, label=f"Reindex {l} row {t}")
            pos = pos0 + t
            lo = max(0, pos - 127)
            for l in range(20, 40):
                win = sw[l - 20][lo - (pos0 - 127): pos - (pos0 - 127) + 1]
                ref = oracle.decode_attention(qq[l - 20][t], kc, ks, 0, lists[model.list_source(l)][t],
                                              win, win.shape[0], SCALE)
                assert attn_rel_err(out[l - 20][t], ref) <= ATTN_TOL, f"layer {l} row {t}"


def test_attn_prefill_without_list():
    # k = 0: window-only rows, clipped at the start of the sequence
    log("attn prefill k=0")
    T, pos0 = 40, 5
    cache = synth.make_entries([64], seed=3, device=DEV)
    q = synth.make_queries(T, 3, device=DEV)
    swa = synth.make_swa(1, T + 127, 3, device=DEV)[0]
    out = torch.empty((T, 16, 512), dtype=torch.float32, device=DEV)
    csa2.csa2_sparse_attn_prefill(q, cache.kv_codes, cache.kv_scale, None, swa, pos0, out,
                                  csa2.attn_workspace(T, 0))
    torch.cuda.synchronize()
    qq, sw, g = h(q), h(swa), h(out)
    for t in (0, 17, T - 1):
        pos = pos0 + t
        lo = max(0, pos - 127)
        win = sw[lo - (pos0 - 127): pos - (pos0 - 127) + 1]
        ref = oracle.decode_attention(qq[t], h(cache.kv_codes), h(cache.kv_scale), 0,
                                      np.zeros(0, np.int32), win, win.shape[0], SCALE)
        assert attn_rel_err(g[t], ref) <= ATTN_TOL


def test_replay_chunk_full_size():
    # the benchmark's shape: the last 128 tokens of a 2^20-token sequence; sampled queries
    n, T = 1 << 20, 128
    pos0 = n - T
    log(f"replay full size n={n} T={T}")
    seed = 12
    cache = synth.make_entries([n], seed=seed, device=DEV)
    q_idx = {l: synth.make_index_queries(T, seed, device=DEV, sub=l) for l in (20,) + model.REINDEX}
    q = torch.stack([synth.make_queries(T, seed, device=DEV, sub=l) for l in range(20, 40)]).contiguous()
    swa = torch.stack([synth.make_swa(1, T + 127, seed, device=DEV, sub=l)[0] for l in range(20, 40)]).contiguous()
    run = model.ReplayChunk(T, n, pos0, device=DEV)
    run.step(cache, q_idx, q, swa)
    torch.cuda.synchronize()
    assert_ws_ok(*run.workspaces())
    codes, scale = h(cache.idx_codes), h(cache.idx_scale)
    kc, ks = h(cache.kv_codes), h(cache.kv_scale)
    pool = h(run.pool)
    lists = {l: h(v) for l, v in run.lists.items()}
    out, qq, sw = h(run.out), h(q), h(swa)
    for t in (0, T - 1):
        vis = pos0 + t + 1
        s = oracle.index_scores(h(q_idx[20])[t], codes[:vis], scale[:vis])
        check_topk(pool[t], s, 16384, label=f"pool row {t}")
        p = pool[t]
        check_topk(lists[20][t], s[p], 512, ids=p, label=f"own row {t}")
        _, r = oracle.reindex_layer(h(q_idx[32])[t], codes, scale, p)
        check_topk(lists[32][t], r, 512, ids=p, label=f"Reindex 32 row {t}")
        pos = pos0 + t
        for l in (20, 27, 32, 39):
            win = sw[l - 20][pos - 127 - (pos0 - 127): pos - (pos0 - 127) + 1]
            ref = oracle.decode_attention(qq[l - 20][t], kc, ks, 0, lists[model.list_source(l)][t],
                                          win, win.shape[0], SCALE)
            assert attn_rel_err(out[l - 20][t], ref) <= ATTN_TOL, f"layer {l} row {t}"
