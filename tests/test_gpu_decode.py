"""GPU parity of the decode path (a1-a6) against the fp64 oracle, through the C ABI.

Small cases compare every output; the workload-sized cases (32 x 32,768 Full decode,
the 16 x 131,072 decoder chain, 4 x 2^20 long decode) run in the launch configuration
the benchmark times and compare sampled rows.  Selections are checked two ways: (1)
bit-exact against the oracle's selection rule applied to the GPU's own fp32 scores, and
(2) against fp64 oracle scores under the gap rule.  Later stages are checked staged: the
oracle is fed the GPU's previous-stage indices.
"""
import math
import sys

import numpy as np
import pytest
import torch

import compressed_sparse_kv_csa2_amd as csa2
import oracle
import synth
from _util import ATTN_TOL, assert_ws_ok, attn_rel_err, check_topk, score_error_bound

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCALE = 1.0 / math.sqrt(512)


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


def run_scan(cache, q_idx, n_cols, cand=None, n_valid=None, topk_ws=None):
    B = q_idx.shape[0]
    scores = torch.empty((B, n_cols), dtype=torch.float32, device=DEV)
    nv = cache.n_entries if n_valid is None else n_valid
    csa2.csa2_index_score(q_idx, cache.idx_codes, cache.idx_scale, cache.seq_base, nv, scores,
                          cand=cand, topk_ws=topk_ws)
    return scores


def run_topk(scores, n_valid, k, cand=None, fused=False, ws=None, with_scores=False):
    B, n = scores.shape
    idx = torch.empty((B, k), dtype=torch.int32, device=DEV)
    so = torch.empty((B, k), dtype=torch.float32, device=DEV) if with_scores else None
    if ws is None and n > 16384:
        ws = csa2.topk_workspace(B, n, k)
    csa2.csa2_topk(scores, n_valid, k, idx, score_out=so, cand=cand, hist_fused=fused, workspace=ws)
    return (idx, so) if with_scores else idx


def run_attn(q, cache, idx, swa, swa_len):
    B = q.shape[0]
    out = torch.empty((B, 16, 512), dtype=torch.float32, device=DEV)
    ws = csa2.attn_workspace(B, 0 if idx is None else idx.shape[1])
    csa2.csa2_sparse_attn_decode(q, cache.kv_codes, cache.kv_scale, cache.seq_base, idx, swa, swa_len,
                                 out, ws, SCALE)
    return out


# --------------------------------------------------------------------------- a1 / a3
@pytest.mark.parametrize("n", [1, 63, 2048, 5000])
def test_scan_scores_within_fp32_bound(n):
    log(f"scan n={n}")
    cache = synth.make_entries([n, 7], seed=100 + n, device=DEV)
    q = synth.make_index_queries(2, 100 + n, device=DEV)
    sc = run_scan(cache, q, max(n, 7) + 3)
    torch.cuda.synchronize()
    codes, scale = h(cache.idx_codes), h(cache.idx_scale)
    for b, (base, cnt) in enumerate([(0, n), (n, 7)]):
        ref = oracle.index_scores(h(q)[b], codes[base:base + cnt], scale[base:base + cnt])
        got = h(sc)[b]
        bound = score_error_bound(h(q)[b], codes[base:base + cnt], scale[base:base + cnt])
        assert np.all(np.abs(got[:cnt] - ref) <= bound)
        assert np.all(np.isneginf(got[cnt:]))


def test_scan_candidate_mode_with_holes():
    log("scan cand")
    n = 9000
    cache = synth.make_entries([n, n], seed=5, device=DEV)
    q = synth.make_index_queries(2, 5, device=DEV)
    rng = np.random.default_rng(5)
    cand = np.stack([np.sort(rng.choice(n, 700, replace=False)) for _ in range(2)]).astype(np.int32)
    cand[1, 650:] = -1
    sc = run_scan(cache, q, 700, cand=torch.from_numpy(cand).to(DEV), n_valid=i32([700, 690]))
    torch.cuda.synchronize()
    codes, scale = h(cache.idx_codes), h(cache.idx_scale)
    for b in range(2):
        ids = cand[b][cand[b] >= 0][: [700, 690][b]]
        ref = oracle.index_scores(h(q)[b], codes[b * n + ids], scale[b * n + ids])
        got = h(sc)[b][: len(ids)]
        assert np.all(np.abs(got - ref) <= score_error_bound(h(q)[b], codes[b * n + ids], scale[b * n + ids]))
    assert np.all(np.isneginf(h(sc)[1][650:]))


# --------------------------------------------------------------------------- a2
def _rand_scores(rng, B, n, tie_frac=0.2):
    s = rng.standard_normal((B, n)).astype(np.float32)
    pool = rng.standard_normal(8).astype(np.float32)
    mask = rng.random((B, n)) < tie_frac
    s[mask] = rng.choice(pool, size=mask.sum())
    s[:, :3] = 0.0
    s[:, 3] = -0.0
    return s


@pytest.mark.parametrize("n,k", [(10, 4), (700, 512), (2048, 512), (16384, 512), (16384, 16384),
                                 (16385, 512), (100_000, 512), (70_000, 16384), (1 << 20, 16384)])
def test_topk_exact_on_gpu_scores(n, k):
    """Same fp32 scores on both sides: the selection must match the oracle bit for bit."""
    log(f"topk n={n} k={k}")
    rng = np.random.default_rng(n + k)
    B = 3
    s = _rand_scores(rng, B, n)
    nv = [n, max(1, n // 3), min(n, k - 1) if k > 1 else 1]
    idx = run_topk(torch.from_numpy(s).to(DEV), i32(nv), k)
    torch.cuda.synchronize()
    g = h(idx)
    for b in range(B):
        want = oracle.topk(s[b].astype(np.float64), k, n_valid=nv[b])
        assert np.array_equal(g[b], want), f"row {b}"


def test_topk_with_candidate_map_and_holes():
    log("topk cand map")
    rng = np.random.default_rng(3)
    n = 16384
    s = _rand_scores(rng, 2, n)
    cand = np.stack([np.sort(rng.choice(10 * n, n, replace=False)) for _ in range(2)]).astype(np.int32)
    cand[1, -100:] = -1
    idx, so = run_topk(torch.from_numpy(s).to(DEV), i32([n, n]), 512,
                       cand=torch.from_numpy(cand).to(DEV), with_scores=True)
    torch.cuda.synchronize()
    for b in range(2):
        keep = cand[b] >= 0
        sel = oracle.topk(np.where(keep, s[b].astype(np.float64), -np.inf), 512)
        assert np.array_equal(h(idx)[b], cand[b][sel])
        assert np.array_equal(h(so)[b], s[b][sel])


def test_topk_fused_histogram_matches_unfused():
    log("topk fused")
    n = 200_000
    cache = synth.make_entries([n, n - 5], seed=8, device=DEV)
    q = synth.make_index_queries(2, 8, device=DEV)
    ws = csa2.topk_workspace(2, n, 16384)
    sc = run_scan(cache, q, n, topk_ws=ws)
    a = run_topk(sc, cache.n_entries, 16384, fused=True, ws=ws)
    b = run_topk(sc, cache.n_entries, 16384, ws=ws)  # workspace came back clean
    c = run_topk(sc, cache.n_entries, 16384, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(b, c)
    for r in range(2):
        assert np.array_equal(h(a)[r], oracle.topk(h(sc)[r].astype(np.float64), 16384,
                                                   n_valid=[n, n - 5][r]))


def test_topk_all_ties_take_lowest_indices():
    log("topk ties")
    n = 50_000
    cache = synth.make_entries([n], seed=9, device=DEV)
    q = torch.zeros((1, 128), dtype=torch.int16, device=DEV)  # every score is 0
    for fused in (False, True):
        ws = csa2.topk_workspace(1, n, 512)
        sc = run_scan(cache, q, n, topk_ws=ws if fused else None)
        idx = run_topk(sc, cache.n_entries, 512, fused=fused, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(h(idx)[0], np.arange(512))


# --------------------------------------------------------------------------- a5 / a6
@pytest.mark.parametrize("k,swa_len", [(512, 128), (37, 5), (0, 128), (64, 0), (512, 0), (2900, 128)])
def test_attention_matches_oracle(k, swa_len):
    log(f"attn k={k} swa={swa_len}")
    n = 3000
    B = 3
    cache = synth.make_entries([n] * B, seed=k + 7, device=DEV)
    q = synth.make_queries(B, k + 7, device=DEV)
    swa = synth.make_swa(B, 128, k + 7, device=DEV)
    rng = np.random.default_rng(k)
    idx_np = np.stack([np.sort(rng.choice(n, k, replace=False)) for _ in range(B)]).astype(np.int32) \
        if k > 0 else np.zeros((B, 0), np.int32)
    if k > 0:
        idx_np[1, ::3] = -1
        idx_np[2, :] = -1 if swa_len > 0 else idx_np[2, :]
    lens = [swa_len, max(0, swa_len - 1), swa_len]
    out = run_attn(q, cache, torch.from_numpy(idx_np).to(DEV) if k > 0 else None, swa, i32(lens))
    torch.cuda.synchronize()
    kc, ks = h(cache.kv_codes), h(cache.kv_scale)
    for b in range(B):
        ref = oracle.decode_attention(h(q)[b], kc, ks, b * n, idx_np[b], h(swa)[b], lens[b], SCALE)
        assert attn_rel_err(h(out)[b], ref) <= ATTN_TOL
        if np.all(ref == 0):
            assert np.all(h(out)[b] == 0)


# --------------------------------------------------------------------------- compositions
def _full_decode(cache, q_idx, q, swa, k=512, pool=None):
    B, N = q_idx.shape[0], int(cache.n_entries.max())
    ws = csa2.topk_workspace(B, N, pool or k)
    sc = run_scan(cache, q_idx, N, topk_ws=ws)
    if pool:
        pidx, pscore = run_topk(sc, cache.n_entries, pool, fused=True, ws=ws, with_scores=True)
        own = run_topk(pscore, i32([pool] * B), k, cand=pidx)
    else:
        pidx, own = None, run_topk(sc, cache.n_entries, k, fused=True, ws=ws)
    out = run_attn(q, cache, own, swa, i32([128] * B))
    return sc, pidx, own, out


def test_c1_tiny_full_decode():
    cfg = synth.CONFIGS["c1_tiny_full"]
    N = synth.entries_for(cfg["ctx"], cfg["ratio"])
    log(f"c1 N={N}")
    cache = synth.make_entries([N], seed=cfg["seed"], device=DEV)
    q_idx = synth.make_index_queries(1, cfg["seed"], device=DEV)
    q = synth.make_queries(1, cfg["seed"], device=DEV)
    swa = synth.make_swa(1, 128, cfg["seed"], device=DEV)
    sc, _, own, out = _full_decode(cache, q_idx, q, swa)
    torch.cuda.synchronize()
    ref_s = oracle.index_scores(h(q_idx)[0], h(cache.idx_codes), h(cache.idx_scale))
    check_topk(h(own)[0], ref_s, 512, label="c1")
    ref_out = oracle.decode_attention(h(q)[0], h(cache.kv_codes), h(cache.kv_scale), 0, h(own)[0],
                                      h(swa)[0], 128, SCALE)
    assert attn_rel_err(h(out)[0], ref_out) <= ATTN_TOL
    # unstaged: the oracle's own selection gives the same output when the sets agree
    ref_idx = oracle.topk(ref_s, 512)
    if np.array_equal(ref_idx, h(own)[0]):
        full = oracle.decode_attention(h(q)[0], h(cache.kv_codes), h(cache.kv_scale), 0, ref_idx,
                                       h(swa)[0], 128, SCALE)
        assert attn_rel_err(h(out)[0], full) <= ATTN_TOL


def test_c2_batched_full_decode():
    cfg = synth.CONFIGS["c2_batched_full"]
    B, N = cfg["B"], synth.entries_for(cfg["ctx"], cfg["ratio"])
    log(f"c2 B={B} N={N}")
    cache = synth.make_entries([N] * B, seed=cfg["seed"], device=DEV)
    q_idx = synth.make_index_queries(B, cfg["seed"], device=DEV)
    q = synth.make_queries(B, cfg["seed"], device=DEV)
    swa = synth.make_swa(B, 128, cfg["seed"], device=DEV)
    sc, _, own, out = _full_decode(cache, q_idx, q, swa)
    torch.cuda.synchronize()
    codes, scale = h(cache.idx_codes), h(cache.idx_scale)
    for b in range(B):
        ref_s = oracle.index_scores(h(q_idx)[b], codes[b * N:(b + 1) * N], scale[b * N:(b + 1) * N])
        check_topk(h(own)[b], ref_s, 512, label=f"c2 row {b}")
        assert np.array_equal(h(own)[b], oracle.topk(h(sc)[b].astype(np.float64), 512))
    for b in (0, 17, 31):
        ref = oracle.decode_attention(h(q)[b], h(cache.kv_codes), h(cache.kv_scale), b * N, h(own)[b],
                                      h(swa)[b], 128, SCALE)
        assert attn_rel_err(h(out)[b], ref) <= ATTN_TOL


def test_c3_decoder_chain():
    cfg = synth.CONFIGS["c3_decoder_chain"]
    B, N, seed = cfg["B"], synth.entries_for(cfg["ctx"], cfg["ratio"]), cfg["seed"]
    log(f"c3 B={B} N={N}")
    cache = synth.make_entries([N] * B, seed=seed, device=DEV)
    layers = list(range(20, 40))
    qi = {l: synth.make_index_queries(B, seed, device=DEV, sub=l) for l in layers
          if oracle.layer_mode(l) in ("full", "reindex")}
    qs = {l: synth.make_queries(B, seed, device=DEV, sub=l) for l in layers}
    sw = {l: synth.make_swa(B, 128, seed, device=DEV, sub=l) for l in layers}
    ws = csa2.topk_workspace(B, N, 16384)
    full_sc = run_scan(cache, qi[20], N, topk_ws=ws)
    pool, pscore = run_topk(full_sc, cache.n_entries, 16384, fused=True, ws=ws, with_scores=True)
    lists, outs, rescores = {}, {}, {}
    lists[20] = run_topk(pscore, i32([16384] * B), 512, cand=pool)
    for l in layers:
        mode = oracle.layer_mode(l)
        if mode == "reindex":
            rescores[l] = run_scan(cache, qi[l], 16384, cand=pool, n_valid=i32([16384] * B))
            lists[l] = run_topk(rescores[l], i32([16384] * B), 512, cand=pool)
        elif mode == "reuse":
            lists[l] = lists[oracle.reuse_source(l)]
        outs[l] = run_attn(qs[l], cache, lists[l], sw[l], i32([128] * B))
    torch.cuda.synchronize()
    codes, scale = h(cache.idx_codes), h(cache.idx_scale)
    kc, ks = h(cache.kv_codes), h(cache.kv_scale)
    for b in (0, 11):
        base = b * N
        ref_full = oracle.index_scores(h(qi[20])[b], codes[base:base + N], scale[base:base + N])
        check_topk(h(pool)[b], ref_full, 16384, label=f"c3 pool {b}")
        p = h(pool)[b]
        check_topk(h(lists[20])[b], ref_full[p], 512, ids=p, label=f"c3 own {b}")
        for l in (24, 36):
            ref_idx, ref_r = oracle.reindex_layer(h(qi[l])[b], codes[base:base + N], scale[base:base + N], p)
            check_topk(h(lists[l])[b], ref_r, 512, ids=p, label=f"c3 reindex {l} {b}")
        for l in (20, 23, 24, 31, 39):
            assert np.array_equal(h(lists[l])[b], h(lists[oracle.reuse_source(l)])[b])
            ref = oracle.decode_attention(h(qs[l])[b], kc, ks, base, h(lists[l])[b], h(sw[l])[b], 128, SCALE)
            assert attn_rel_err(h(outs[l])[b], ref) <= ATTN_TOL, f"layer {l} row {b}"


def test_c4_long_decode_step():
    cfg = synth.CONFIGS["c4_long_decode"]
    B, N, seed = cfg["B"], cfg["ctx"] // cfg["ratio"], cfg["seed"]
    log(f"c4 B={B} N={N}")
    cache = synth.make_entries([N] * B, seed=seed, device=DEV)
    q_full = synth.make_index_queries(B, seed, device=DEV, sub=20)
    q_re = synth.make_index_queries(B, seed, device=DEV, sub=24)
    q = synth.make_queries(B, seed, device=DEV, sub=24)
    swa = synth.make_swa(B, 128, seed, device=DEV, sub=24)
    ws = csa2.topk_workspace(B, N, 16384)
    sc = run_scan(cache, q_full, N, topk_ws=ws)
    pool = run_topk(sc, cache.n_entries, 16384, fused=True, ws=ws)
    rs = run_scan(cache, q_re, 16384, cand=pool, n_valid=i32([16384] * B))
    idx = run_topk(rs, i32([16384] * B), 512, cand=pool)
    out = run_attn(q, cache, idx, swa, i32([128] * B))
    torch.cuda.synchronize()
    codes, scale = h(cache.idx_codes), h(cache.idx_scale)
    for b in (0, B - 1):
        base = b * N
        log(f"c4 oracle row {b}")
        ref_s = oracle.index_scores(h(q_full)[b], codes[base:base + N], scale[base:base + N])
        check_topk(h(pool)[b], ref_s, 16384, label=f"c4 pool {b}")
        assert np.array_equal(h(pool)[b], oracle.topk(h(sc)[b].astype(np.float64), 16384))
        p = h(pool)[b]
        _, ref_r = oracle.reindex_layer(h(q_re)[b], codes[base:base + N], scale[base:base + N], p)
        check_topk(h(idx)[b], ref_r, 512, ids=p, label=f"c4 reindex {b}")
        ref = oracle.decode_attention(h(q)[b], h(cache.kv_codes), h(cache.kv_scale), base, h(idx)[b],
                                      h(swa)[b], 128, SCALE)
        assert attn_rel_err(h(out)[b], ref) <= ATTN_TOL


def test_c4_bench_call_sequence():
    """The benchmark's c4 step exactly: input set 0 of its rotation (layer 20's index query,
    layer 24's index query, layer 24's query and window), csa2_select_chain (Full scan of
    4 x 2^20 entries, pool 16,384, one Reindex layer's top-512, no own list) on the chain
    workspace, then csa2_sparse_attn_decode over the Reindex list.  The pool and the Reindex
    list against fp64 oracle scores, rows 0 and 3's attention against the oracle, and the
    per-layer calls (csa2_index_topk for the pool, then over the pool) give the same lists."""
    cfg = synth.CONFIGS["c4_long_decode"]
    B, N, seed = cfg["B"], cfg["ctx"] // cfg["ratio"], cfg["seed"]
    log(f"c4 bench sequence B={B} N={N}")
    cache = synth.make_entries([N] * B, seed=seed, device=DEV)
    q_full = synth.make_index_queries(B, seed, device=DEV, sub=20)
    q_re = synth.make_index_queries(B, seed, device=DEV, sub=24)
    q = synth.make_queries(B, seed, device=DEV, sub=24)
    swa = synth.make_swa(B, 128, seed, device=DEV, sub=24)
    swa_len = i32([128] * B)
    cws = csa2.select_chain_workspace(B, N, 16384)
    pool = torch.empty((B, 16384), dtype=torch.int32, device=DEV)
    re_out = torch.empty((1, B, 512), dtype=torch.int32, device=DEV)
    csa2.csa2_select_chain(q_full, cache.idx_codes, cache.idx_scale, cache.seq_base, cache.n_entries, N,
                           pool, cws, k=512, q_re=q_re[None].contiguous(), re_out=re_out)
    out = torch.empty((B, 16, 512), dtype=torch.float32, device=DEV)
    aws = csa2.attn_workspace(B, 512)
    csa2.csa2_sparse_attn_decode(q, cache.kv_codes, cache.kv_scale, cache.seq_base, re_out[0], swa,
                                 swa_len, out, aws, softmax_scale=SCALE)
    # the per-layer calls on the same inputs
    fws = csa2.index_topk_workspace(B, N, 16384)
    rws = csa2.index_topk_workspace(B, 16384, 512)
    pool2 = torch.empty_like(pool)
    idx2 = torch.empty((B, 512), dtype=torch.int32, device=DEV)
    csa2.csa2_index_topk(q_full, cache.idx_codes, cache.idx_scale, cache.seq_base, cache.n_entries, 16384,
                         pool2, fws, N)
    csa2.csa2_index_topk(q_re, cache.idx_codes, cache.idx_scale, cache.seq_base, i32([16384] * B), 512,
                         idx2, rws, 16384, cand=pool2)
    torch.cuda.synchronize()
    assert_ws_ok(cws, fws, rws)
    assert torch.equal(pool, pool2) and torch.equal(re_out[0], idx2), "per-layer calls differ"
    codes, scale = h(cache.idx_codes), h(cache.idx_scale)
    for b in (0, B - 1):
        base = b * N
        log(f"c4 bench sequence oracle row {b}")
        s = oracle.index_scores(h(q_full)[b], codes[base:base + N], scale[base:base + N])
        check_topk(h(pool)[b], s, 16384, label=f"pool {b}")
        p = h(pool)[b]
        _, ref_r = oracle.reindex_layer(h(q_re)[b], codes[base:base + N], scale[base:base + N], p)
        check_topk(h(re_out)[0][b], ref_r, 512, ids=p, label=f"reindex {b}")
        ref = oracle.decode_attention(h(q)[b], h(cache.kv_codes), h(cache.kv_scale), base, h(re_out)[0][b],
                                      h(swa)[b], 128, SCALE)
        assert attn_rel_err(h(out)[b], ref) <= ATTN_TOL, f"attention row {b}"


def test_decode_is_deterministic():
    log("determinism")
    cache = synth.make_entries([40_000, 40_000], seed=13, device=DEV)
    q_idx = synth.make_index_queries(2, 13, device=DEV)
    q = synth.make_queries(2, 13, device=DEV)
    swa = synth.make_swa(2, 128, 13, device=DEV)
    r1 = _full_decode(cache, q_idx, q, swa, pool=16384)
    r2 = _full_decode(cache, q_idx, q, swa, pool=16384)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


def test_empty_and_short_rows():
    log("empty rows")
    cache = synth.make_entries([0, 300, 20_000], seed=14, device=DEV)
    B = 3
    q_idx = synth.make_index_queries(B, 14, device=DEV)
    q = synth.make_queries(B, 14, device=DEV)
    swa = synth.make_swa(B, 128, 14, device=DEV)
    N = 20_000
    sc = run_scan(cache, q_idx, N)
    idx = run_topk(sc, cache.n_entries, 512)
    out = run_attn(q, cache, idx, swa, i32([0, 128, 3]))
    torch.cuda.synchronize()
    g = h(idx)
    assert np.all(g[0] == -1)
    assert np.array_equal(g[1][:300], np.arange(300)) and np.all(g[1][300:] == -1)
    assert np.all(h(out)[0] == 0)
    kc, ks = h(cache.kv_codes), h(cache.kv_scale)
    for b, base, ln in [(1, 0, 128), (2, 300, 3)]:
        ref = oracle.decode_attention(h(q)[b], kc, ks, base, g[b], h(swa)[b], ln, SCALE)
        assert attn_rel_err(h(out)[b], ref) <= ATTN_TOL
