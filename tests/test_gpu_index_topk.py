"""GPU parity of csa2_index_topk (scan + top-k in one call) through the C ABI.

Its selection is compared (1) bit for bit with the oracle's selection rule applied to the
GPU's own fp32 scores from csa2_index_score (both calls run the same scan arithmetic),
(2) with csa2_index_score + csa2_topk, output for output, and (3) against fp64 oracle
scores under the gap rule.  The workspace must come back ready for the next call: the
status block reports no error and the per-row counters return to zero.
"""
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    csa2.load_library()


def h(t):
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def i32(x):
    return torch.tensor(x, dtype=torch.int32, device=DEV)


def fused(cache, q_idx, n_cols, k, n_valid=None, cand=None, ws=None):
    B = q_idx.shape[0]
    nv = cache.n_entries if n_valid is None else n_valid
    ws = csa2.index_topk_workspace(B, n_cols, k) if ws is None else ws
    idx = torch.full((B, k), -7, dtype=torch.int32, device=DEV)
    so = torch.full((B, k), 7.0, dtype=torch.float32, device=DEV)
    csa2.csa2_index_topk(q_idx, cache.idx_codes, cache.idx_scale, cache.seq_base, nv, k, idx, ws,
                         n_cols, score_out=so, cand=cand)
    return idx, so, ws


def two_step(cache, q_idx, n_cols, k, n_valid=None, cand=None):
    B = q_idx.shape[0]
    nv = cache.n_entries if n_valid is None else n_valid
    sc = torch.empty((B, n_cols), dtype=torch.float32, device=DEV)
    csa2.csa2_index_score(q_idx, cache.idx_codes, cache.idx_scale, cache.seq_base, nv, sc, cand=cand)
    idx = torch.empty((B, k), dtype=torch.int32, device=DEV)
    so = torch.empty((B, k), dtype=torch.float32, device=DEV)
    ws = csa2.topk_workspace(B, n_cols, k) if n_cols > 16384 else None
    csa2.csa2_topk(sc, nv, k, idx, score_out=so, cand=cand, workspace=ws)
    return sc, idx, so


def ws_clean(ws, B, slow=None):
    """Status block: no error bits (and, when given, the number of rows that took the
    second scan); the per-row counters that follow it (64 bytes per row from byte 256)
    back to zero."""
    bits, n_slow = csa2.csa2_workspace_status(ws)
    assert bits == 0, f"workspace error bits {bits:#x}"
    if slow is not None:
        assert n_slow == slow, f"{n_slow} rows re-scanned, expected {slow}"
    w = h(ws)
    rows = min(B, 16)
    assert not w[256:256 + rows * 64].any(), "per-row counters not reset"


def same_as_two_step(cache, q_idx, n_cols, k, n_valid=None, cand=None, rows=None):
    idx, so, ws = fused(cache, q_idx, n_cols, k, n_valid, cand)
    sc, idx2, so2 = two_step(cache, q_idx, n_cols, k, n_valid, cand)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2), "differs from csa2_index_score + csa2_topk"
    assert torch.equal(so, so2), "scores of the selection differ"
    nv = h(cache.n_entries if n_valid is None else n_valid)
    s = h(sc)
    c = None if cand is None else h(cand)
    for b in (range(q_idx.shape[0]) if rows is None else rows):
        if c is None:
            want = oracle.topk(s[b].astype(np.float64), k, n_valid=int(nv[b]))
            assert np.array_equal(h(idx)[b], want), f"row {b}"
        else:
            keep = np.arange(n_cols) < nv[b]
            keep &= c[b] >= 0
            sel = oracle.topk(np.where(keep, s[b].astype(np.float64), -np.inf), k)
            want = np.where(sel >= 0, c[b][np.maximum(sel, 0)], -1)
            assert np.array_equal(h(idx)[b], want), f"row {b}"
    return idx, so, ws


@pytest.mark.parametrize("n,k", [(1, 4), (700, 512), (2048, 512), (5000, 512), (33_000, 512),
                                 (70_000, 16384), (131_072 + 77, 16384), (16384, 16384)])
def test_full_matches_two_step_and_oracle_rule(n, k):
    log(f"index_topk full n={n} k={k}")
    B = 3
    lens = [n, max(1, n // 3), max(1, n - 129)]
    cache = synth.make_entries(lens, seed=200 + n % 97, device=DEV)
    q = synth.make_index_queries(B, 200 + n % 97, device=DEV)
    _, _, ws = same_as_two_step(cache, q, n, k)
    ws_clean(ws, B)


def test_full_against_fp64_oracle_scores():
    log("index_topk gap rule")
    n = 20_000
    cache = synth.make_entries([n, n - 11], seed=31, device=DEV)
    q = synth.make_index_queries(2, 31, device=DEV)
    idx, _, _ = fused(cache, q, n, 512)
    torch.cuda.synchronize()
    codes, scale = h(cache.idx_codes), h(cache.idx_scale)
    for b, (base, cnt) in enumerate([(0, n), (n, n - 11)]):
        ref = oracle.index_scores(h(q)[b], codes[base:base + cnt], scale[base:base + cnt])
        check_topk(h(idx)[b], ref, 512, label=f"row {b}")


def test_reindex_candidates_with_holes():
    log("index_topk reindex")
    n, P = 40_000, 16384
    cache = synth.make_entries([n, n, n], seed=32, device=DEV)
    q = synth.make_index_queries(3, 32, device=DEV)
    rng = np.random.default_rng(32)
    cand = np.stack([np.sort(rng.choice(n, P, replace=False)) for _ in range(3)]).astype(np.int32)
    cand[1, 5000:5100] = -1
    cand[2, P - 300:] = -1
    cand_t = torch.from_numpy(cand).to(DEV)
    _, _, ws = same_as_two_step(cache, q, P, 512, n_valid=i32([P, P, P - 17]), cand=cand_t)
    ws_clean(ws, 3)


def test_empty_rows_and_more_k_than_columns():
    log("index_topk empty / short")
    cache = synth.make_entries([3000, 3000, 3000], seed=33, device=DEV)
    q = synth.make_index_queries(3, 33, device=DEV)
    idx, so, ws = fused(cache, q, 3000, 600, n_valid=i32([0, 3000, 450]))
    torch.cuda.synchronize()
    g, s = h(idx), h(so)
    assert np.all(g[0] == -1) and np.all(np.isneginf(s[0]))
    assert np.all(g[2][:450] == np.arange(450)) and np.all(g[2][450:] == -1)
    assert np.all(np.isneginf(s[2][450:]))
    ws_clean(ws, 3)


def test_all_ties_take_lowest_columns():
    log("index_topk ties")
    n = 50_000
    cache = synth.make_entries([n], seed=34, device=DEV)
    q = torch.zeros((1, 128), dtype=torch.int16, device=DEV)  # every score is 0
    for k in (512, 16384):
        idx, _, ws = fused(cache, q, n, k)
        torch.cuda.synchronize()
        assert np.array_equal(h(idx)[0], np.arange(k))
        ws_clean(ws, 1)


@pytest.mark.parametrize("dims,k", [(1, 512), (1, 16384), (3, 512), (3, 16384)])
def test_ties_at_the_threshold(dims, k):
    """Unit scales and a query with few non-zero components: scores take few distinct
    values, so the k-th score is shared by many columns across many workgroups (with one
    component: thousands, the massive-tie path; with three: a handful)."""
    log(f"index_topk threshold ties dims={dims} k={k}")
    n = 300_000
    cache = synth.make_entries([n, n - 1000], seed=40 + dims, device=DEV)
    cache.idx_scale.fill_(1.0)
    q = torch.zeros((2, 128), dtype=torch.float32)
    q[:, :dims] = torch.tensor([1.0, 0.5, 0.25][:dims])
    q_bits = q.to(torch.bfloat16).view(torch.int16).to(DEV)
    _, _, ws = same_as_two_step(cache, q_bits, n, k)
    ws_clean(ws, 2)


def test_workspace_reuse_is_deterministic():
    log("index_topk reuse")
    n = 100_000
    caches = [synth.make_entries([n, n], seed=35 + i, device=DEV) for i in range(2)]
    qs = [synth.make_index_queries(2, 35 + i, device=DEV) for i in range(2)]
    ws = csa2.index_topk_workspace(2, n, 16384)
    outs = []
    for it in range(4):
        idx, _, _ = fused(caches[it % 2], qs[it % 2], n, 16384, ws=ws)
        outs.append(idx.clone())
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[2]) and torch.equal(outs[1], outs[3])
    assert not torch.equal(outs[0], outs[1])
    ws_clean(ws, 2)


def test_segment_overflow_takes_the_second_scan():
    """4,000 entries inside the first 16,384-column segment of row 0 score far above every
    other entry.  The segment keeps only its expected share of the top-k plus six standard
    deviations (about 3,000 keys), every kept key wins, so the selection cannot be sure of
    the segment's share: it scans the row again keeping every key, and the result is still
    exact (and counted in the status block)."""
    log("index_topk forced second scan")
    n, k = 100_000, 16384
    cache = synth.make_entries([n, n], seed=45, device=DEV)
    cols = torch.arange(1000, 5000, device=DEV)
    cache.idx_codes[cols] = 0x77           # every value 6
    cache.idx_scale[cols] = 1000.0
    q = torch.ones((2, 128), dtype=torch.float32).to(torch.bfloat16).view(torch.int16).to(DEV)
    ws = csa2.index_topk_workspace(2, n, k)
    idx, so, _ = fused(cache, q, n, k, ws=ws)
    _, idx2, so2 = two_step(cache, q, n, k)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(so, so2)
    ws_clean(ws, 2, slow=1)                # only row 0 holds the planted entries
    s0 = oracle.index_scores(h(q)[0], h(cache.idx_codes)[:n], h(cache.idx_scale)[:n])
    check_topk(h(idx)[0], s0, k, label="row 0")


def test_ragged_rows_mix_sampled_and_unsampled():
    """Rows with every valid key kept (<= 32,768 columns) and sampled rows in one call, with
    lengths that end inside a chunk, exactly at chunk ends and at zero."""
    log("index_topk ragged rows")
    lens = [1, 1920, 1921, 32_768, 32_769, 65_536 + 7, 3 * 1920 * 17, 0]
    cache = synth.make_entries([max(1, x) for x in lens], seed=46, device=DEV)
    q = synth.make_index_queries(len(lens), 46, device=DEV)
    n_cols = max(lens)
    for k in (512, 16384):
        _, _, ws = same_as_two_step(cache, q, n_cols, k, n_valid=i32(lens))
        ws_clean(ws, len(lens))


def test_long_decode_pool_and_reindex_at_full_size():
    """4 x 2^20 Full scan -> pool of 16,384 -> Reindex top-512, as the benchmark runs it."""
    cfg = synth.CONFIGS["c4_long_decode"]
    B, N = cfg["B"], 1 << 20
    log(f"index_topk 2^20 B={B}")
    cache = synth.make_entries([N] * B, seed=cfg["seed"], device=DEV)
    q_full = synth.make_index_queries(B, cfg["seed"], device=DEV)
    q_re = synth.make_index_queries(B, cfg["seed"] + 1000, device=DEV)
    pool, _, ws = same_as_two_step(cache, q_full, N, 16384, rows=[0, 3])
    ws_clean(ws, B)
    same_as_two_step(cache, q_re, 16384, 512, n_valid=i32([16384] * B), cand=pool)


def test_many_rows_of_2_20():
    """5 x 2^20 columns: more rows than the c4 batch, chunks claimed across all of them."""
    B, N = 5, 1 << 20
    log(f"index_topk split B={B}")
    cache = synth.make_entries([N] * B, seed=36, device=DEV)
    q = synth.make_index_queries(B, 36, device=DEV)
    _, _, ws = same_as_two_step(cache, q, N, 512, rows=[0, 4])
    ws_clean(ws, B)


def test_row_longer_than_the_filtered_selection():
    """A row of more than 2,048 chunks of 1,920 columns takes the scan-then-top-k path
    inside the call."""
    n = 256 * 16384 + 5000
    log(f"index_topk long row n={n}")
    cache = synth.make_entries([n], seed=37, device=DEV)
    q = synth.make_index_queries(1, 37, device=DEV)
    same_as_two_step(cache, q, n, 16384)


# --------------------------------------------------------------------------- chained selections
def chain(cache, q_full, n_cols, pool_k, k, q_re=None, own=True, ws=None):
    B = q_full.shape[0]
    ws = csa2.select_chain_workspace(B, n_cols, pool_k) if ws is None else ws
    pool = torch.full((B, pool_k), -7, dtype=torch.int32, device=DEV)
    pscore = torch.full((B, pool_k), 7.0, dtype=torch.float32, device=DEV)
    own_out = torch.full((B, k), -7, dtype=torch.int32, device=DEV) if own else None
    n_re = 0 if q_re is None else q_re.shape[0]
    re_out = torch.full((n_re, B, k), -7, dtype=torch.int32, device=DEV) if n_re else None
    re_sc = torch.full((n_re, B, k), 7.0, dtype=torch.float32, device=DEV) if n_re else None
    csa2.csa2_select_chain(q_full, cache.idx_codes, cache.idx_scale, cache.seq_base, cache.n_entries,
                           n_cols, pool, ws, k=k, pool_score_out=pscore, own_out=own_out,
                           q_re=q_re, re_out=re_out, re_score_out=re_sc)
    return pool, pscore, own_out, re_out, re_sc, ws


def separate(cache, q_full, n_cols, pool_k, k, q_re=None):
    B = q_full.shape[0]
    pool, pscore, _ = fused(cache, q_full, n_cols, pool_k)
    pool_n = (pool >= 0).sum(dim=1, dtype=torch.int32)
    own = torch.empty((B, k), dtype=torch.int32, device=DEV)
    csa2.csa2_topk(pscore, pool_n, k, own, cand=pool)
    res = []
    for r in range(0 if q_re is None else q_re.shape[0]):
        idx, sc, _ = fused(cache, q_re[r].contiguous(), pool_k, k, n_valid=pool_n, cand=pool)
        res.append((idx, sc))
    return pool, pscore, pool_n, own, res


def check_chain(cache, q_full, n_cols, pool_k, k, q_re=None, rows=None, ws=None):
    pool, pscore, own, re_out, re_sc, ws = chain(cache, q_full, n_cols, pool_k, k, q_re, ws=ws)
    pool2, pscore2, pool_n, own2, res2 = separate(cache, q_full, n_cols, pool_k, k, q_re)
    torch.cuda.synchronize()
    assert torch.equal(pool, pool2) and torch.equal(pscore, pscore2), "pool differs"
    assert torch.equal(own, own2), "own top-k differs"
    for r, (idx2, sc2) in enumerate(res2):
        assert torch.equal(re_out[r], idx2), f"Reindex layer {r} differs"
        assert torch.equal(re_sc[r], sc2), f"Reindex layer {r} scores differ"
    # the own top-k against the oracle's rule on the pool's scores
    P, S, N, O = h(pool), h(pscore), h(pool_n), h(own)
    for b in (range(q_full.shape[0]) if rows is None else rows):
        sel = oracle.topk(S[b].astype(np.float64), k, n_valid=int(N[b]))
        want = np.where(sel >= 0, P[b][np.maximum(sel, 0)], -1)
        assert np.array_equal(O[b], want), f"own top-k row {b}"
    ws_clean(ws, q_full.shape[0])
    return pool, own, re_out


@pytest.mark.parametrize("n,pool_k,n_re", [(70_000, 16384, 2), (5000, 600, 1), (300_000, 16384, 4)])
def test_chain_matches_separate_calls(n, pool_k, n_re):
    log(f"select_chain n={n} pool={pool_k} re={n_re}")
    B = 3
    lens = [n, max(1, n // 7), max(1, n - 333)]
    cache = synth.make_entries(lens, seed=50 + n_re, device=DEV)
    q = synth.make_index_queries(B, 50 + n_re, device=DEV)
    q_re = torch.stack([synth.make_index_queries(B, 60 + n_re + r, device=DEV)
                        for r in range(n_re)]).contiguous()
    check_chain(cache, q, n, pool_k, 512, q_re)


def test_chain_with_ties():
    """Zero queries: every score ties, in the pool and in every Reindex layer."""
    log("select_chain ties")
    n = 40_000
    cache = synth.make_entries([n, n], seed=70, device=DEV)
    q = torch.zeros((2, 128), dtype=torch.int16, device=DEV)
    q_re = torch.zeros((2, 2, 128), dtype=torch.int16, device=DEV)
    pool, own, re_out = check_chain(cache, q, n, 16384, 512, q_re)
    assert np.array_equal(h(pool)[0], np.arange(16384))
    assert np.array_equal(h(own)[1], np.arange(512))
    assert np.array_equal(h(re_out)[1][0], np.arange(512))


def check_chain_fp64(cache, q_full, q_re, pool, own, re_out, rows, pool_k=16384, k=512):
    """The chain's pool, own top-k and every Reindex list against fp64 oracle scores (gap
    rule): the pool and own top-k over the row's scores, each Reindex list over the re-scores
    of the pool's entries."""
    codes, scale = h(cache.idx_codes), h(cache.idx_scale)
    bases, lens = h(cache.seq_base), h(cache.n_entries)
    P, R = h(pool), None if re_out is None else h(re_out)
    for b in rows:
        base, n = int(bases[b]), int(lens[b])
        log(f"chain fp64 row {b}")
        s = oracle.index_scores(h(q_full)[b], codes[base:base + n], scale[base:base + n])
        check_topk(P[b], s, pool_k, label=f"pool row {b}")
        if own is not None:
            check_topk(h(own)[b], s, k, label=f"own row {b}")
        pv = P[b][P[b] >= 0]
        for r in range(0 if q_re is None else q_re.shape[0]):
            sr = oracle.index_scores(h(q_re)[r][b], codes[base + pv], scale[base + pv])
            check_topk(R[r][b], sr, k, ids=pv, label=f"Reindex {r} row {b}")


def test_chain_long_decode_at_full_size():
    """4 x 2^20 Full scan -> pool 16,384 -> own top-512 and one Reindex layer, three calls
    on one workspace."""
    cfg = synth.CONFIGS["c4_long_decode"]
    B, N = cfg["B"], 1 << 20
    log(f"select_chain 2^20 B={B}")
    cache = synth.make_entries([N] * B, seed=cfg["seed"], device=DEV)
    ws = csa2.select_chain_workspace(B, N, 16384)
    for rep in range(3):
        q = synth.make_index_queries(B, cfg["seed"] + rep, device=DEV)
        q_re = synth.make_index_queries(B, cfg["seed"] + 1000 + rep, device=DEV)[None].contiguous()
        pool, own, re_out = check_chain(cache, q, N, 16384, 512, q_re, rows=[0, 3], ws=ws)
    check_chain_fp64(cache, q, q_re, pool, own, re_out, rows=[0, 3])


def test_chain_decoder_layer_chain_at_full_size():
    """16 x 131,072: one Full layer (pool + own top-512) and four Reindex layers."""
    cfg = synth.CONFIGS["c3_decoder_chain"]
    B, N = cfg["B"], cfg["ctx"] // cfg["ratio"]
    log(f"select_chain chain B={B} N={N}")
    cache = synth.make_entries([N] * B, seed=cfg["seed"], device=DEV)
    q = synth.make_index_queries(B, cfg["seed"], device=DEV)
    q_re = torch.stack([synth.make_index_queries(B, cfg["seed"] + 10 + r, device=DEV)
                        for r in range(4)]).contiguous()
    pool, own, re_out = check_chain(cache, q, N, 16384, 512, q_re, rows=[0, 15])
    check_chain_fp64(cache, q, q_re, pool, own, re_out, rows=[0, 15])
