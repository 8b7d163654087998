"""GPU parity of csa2_replay_select (the decoder replay's Full-layer selections: the causal
MFMA score matrix of a chunk of queries, then the filtered selection on it) against the
oracle: per query, the pool of its best visible entries and its own top-k inside that pool,
judged on fp64 oracle scores by the top-k parity rule; each pool's valid count; causal
visibility at ratios 1, 2 and 4; chunks of more than one 128-row block; the start of a
sequence (pools padded with -1); a sequence with no entries; and a row forced onto the
selection's slow path."""
import sys

import numpy as np
import pytest
import torch

import compressed_sparse_kv_csa2_amd as csa2
import oracle
import synth
from _util import check_topk

pytestmark = pytest.mark.gpu
DEV = "cuda"


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def h(t):
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def run(cache, q, n, ratio, pos0, pool_k, k, ws=None):
    T = q.shape[0]
    pool = torch.full((T, pool_k), -7, dtype=torch.int32, device=DEV)
    own = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    pn = torch.full((T,), -7, dtype=torch.int32, device=DEV)
    if ws is None:
        ws = csa2.replay_select_workspace(T, n, pool_k)
    csa2.csa2_replay_select(q, cache.idx_codes, cache.idx_scale, n, ratio, pos0, pool, ws, k=k,
                            own_out=own, pool_n_out=pn)
    torch.cuda.synchronize()
    return pool, own, pn, ws


def visible(pos, ratio, n):
    return min(n, (pos + 1) // ratio)


def check_rows(cache, q, n, ratio, pos0, pool_k, k, pool, own, pn, rows):
    codes, scale, qq = h(cache.idx_codes), h(cache.idx_scale), h(q)
    pool, own, pn = h(pool), h(own), h(pn)
    for t in rows:
        vis = visible(pos0 + t, ratio, n)
        assert pn[t] == min(vis, pool_k), f"row {t}: pool count {pn[t]}, want {min(vis, pool_k)}"
        s = oracle.index_scores(qq[t], codes[:vis], scale[:vis])
        check_topk(pool[t], s, pool_k, label=f"pool row {t}")
        p = pool[t][pool[t] >= 0]
        check_topk(own[t], s[p] if len(p) else np.zeros(0), k, ids=p, label=f"own row {t}")


@pytest.mark.parametrize("n,ratio,T,pos0,pool_k,k", [
    (20000, 1, 200, 19800, 16384, 512),   # every key kept; two 128-row blocks
    (60000, 2, 150, 100000, 4096, 512),   # segments cut (rows of 50,000 entries) at ratio 2
    (3000, 1, 64, 0, 16384, 512),         # start of a sequence: pools shorter than pool_k
    (5000, 4, 40, 100, 100, 50),          # ratio 4, tiny rows
])
def test_replay_select_matches_oracle(n, ratio, T, pos0, pool_k, k):
    log(f"replay_select n={n} ratio={ratio} T={T} pos0={pos0} pool={pool_k} k={k}")
    seed = 70 + ratio
    cache = synth.make_entries([n], seed=seed, device=DEV)
    q = synth.make_index_queries(T, seed, device=DEV)
    pool, own, pn, ws = run(cache, q, n, ratio, pos0, pool_k, k)
    assert csa2.csa2_workspace_status(ws) == (0, 0)
    rows = sorted({0, 1, 31, 32, 63, 64, 127, 128, T - 1} & set(range(T)) | set(range(0, T, 23)))
    check_rows(cache, q, n, ratio, pos0, pool_k, k, pool, own, pn, rows)
    # a second call on the same workspace gives the same lists
    pool2, own2, pn2, _ = run(cache, q, n, ratio, pos0, pool_k, k, ws=ws)
    assert torch.equal(pool, pool2) and torch.equal(own, own2) and torch.equal(pn, pn2)


def test_replay_select_without_entries():
    log("replay_select n=0")
    cache = synth.make_entries([16], seed=3, device=DEV)
    q = synth.make_index_queries(3, 3, device=DEV)
    pool, own, pn, _ = run(cache, q, 0, 1, 10, 64, 8)
    assert (pool == -1).all() and (own == -1).all() and (pn == 0).all()


def test_replay_select_slow_path():
    """4,000 entries score far above the rest for every query (all-ones queries): the
    segments holding them keep only their expected share, every kept key wins, so each row
    is selected again from every score (counted in the status block).  Equal scores go to
    the lower entry: the pool is exactly the first 2,048 planted entries."""
    log("replay_select forced slow path")
    n, T, pool_k, k = 131072, 4, 2048, 512
    cache = synth.make_entries([n], seed=45, device=DEV)
    cols = torch.arange(1000, 5000, device=DEV)
    cache.idx_codes[cols] = 0x77           # every value 6
    cache.idx_scale[cols] = 1000.0
    q = torch.ones((T, 128), dtype=torch.float32).to(torch.bfloat16).view(torch.int16).to(DEV)
    pool, own, pn, ws = run(cache, q, n, 1, n, pool_k, k)
    assert csa2.csa2_workspace_status(ws) == (0, T)
    want = np.arange(1000, 1000 + pool_k)
    for t in range(T):
        assert np.array_equal(h(pool)[t], want), f"row {t}"
        assert np.array_equal(h(own)[t], want[:k]), f"own row {t}"
    check_rows(cache, q, n, 1, n, pool_k, k, pool, own, pn, [0])
