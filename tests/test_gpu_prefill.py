"""GPU parity of the prefill chunk (a7 MFMA scoring, a8 per-query top-k + attention)
against the fp64 oracle, through the C ABI."""
import math
import sys

import numpy as np
import pytest
import torch

import compressed_sparse_kv_csa2_amd as csa2
import oracle
import synth
from _util import ATTN_TOL, attn_rel_err, check_topk

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


def run_prefill(cache, q_idx, q, swa, n_entries, ratio, pos0, k):
    T = q_idx.shape[0]
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    out = torch.empty((T, 16, 512), dtype=torch.float32, device=DEV)
    ws = csa2.prefill_workspace(T, n_entries, k)
    csa2.csa2_prefill_chunk(q_idx, q, cache.idx_codes, cache.idx_scale, cache.kv_codes, cache.kv_scale,
                            n_entries, ratio, pos0, k, swa, idx, out, ws, SCALE)
    return idx, out


def check_rows(cache, q_idx, q, swa, n_entries, ratio, pos0, k, idx, out, rows):
    ic, isc = h(cache.idx_codes), h(cache.idx_scale)
    kc, ks = h(cache.kv_codes), h(cache.kv_scale)
    qi, qq, sw = h(q_idx), h(q), h(swa)
    keys = oracle.dequant_index_keys(ic[:n_entries])
    kscale = isc[:n_entries].astype(np.float64)
    g_idx, g_out = h(idx), h(out)
    for t in rows:
        p = pos0 + t
        n_t = oracle.visible_entries(p, ratio, n_entries)
        s = kscale[:n_t] * (keys[:n_t] @ oracle.formats.bf16_decode(qi[t]))
        check_topk(g_idx[t], s, k, label=f"prefill row {t}")
        lo = max(0, p - 127)
        win = sw[lo - (pos0 - 127): p - (pos0 - 127) + 1]
        ref = oracle.decode_attention(qq[t], kc, ks, 0, g_idx[t], win, win.shape[0], SCALE)
        assert attn_rel_err(g_out[t], ref) <= ATTN_TOL, f"row {t}"


def _case(N, ratio, T, pos0, k, seed, zero_q=False):
    cache = synth.make_entries([N], seed=seed, device=DEV)
    q_idx = synth.make_index_queries(T, seed, device=DEV)
    if zero_q:
        q_idx.zero_()
    q = synth.make_queries(T, seed, device=DEV)
    swa = synth.make_swa(1, T + 127, seed, device=DEV)[0]
    idx, out = run_prefill(cache, q_idx, q, swa, N, ratio, pos0, k)
    torch.cuda.synchronize()
    return cache, q_idx, q, swa, idx, out


@pytest.mark.parametrize("N,ratio,T,pos0,k", [
    (300, 2, 40, 560, 16),        # tail of a short context
    (5000, 2, 130, 9870, 512),    # several tiles, ragged row block
    (9000, 1, 64, 0, 512),        # start of a sequence: rows see < k entries, window clipped
    (20000, 2, 200, 39800, 100),  # k not a power of two
    (12000, 2, 24, 23000, 2048),  # a row's entry ids staged in several rounds
    (6000, 2, 330, 11660, 256),   # two row blocks, the second ragged inside a wave's row sets
    (8192, 4, 300, 32468, 512),   # V4-style 4:1 compression: one entry per four tokens
    (3000, 4, 64, 0, 512),        # 4:1 from the start of a sequence: rows see 0..16 entries
    (5003, 2, 50, 9956, 512),     # entry count not a multiple of 4: last rows see every entry
    (301, 1, 20, 281, 16),        # likewise, a single tile row block
])
def test_prefill_all_rows(N, ratio, T, pos0, k):
    log(f"prefill N={N} ratio={ratio} T={T} pos0={pos0} k={k}")
    cache, q_idx, q, swa, idx, out = _case(N, ratio, T, pos0, k, seed=N + T)
    check_rows(cache, q_idx, q, swa, N, ratio, pos0, k, idx, out, range(T))


def test_prefill_sampled_threshold_rows():
    # every row sees >= 98,304 entries and k = 512: the threshold comes from a 1-in-4 sample
    log("prefill sampled threshold")
    N, T, pos0, k = 100000, 64, 99000, 512
    cache, q_idx, q, swa, idx, out = _case(N, 1, T, pos0, k, seed=77)
    check_rows(cache, q_idx, q, swa, N, 1, pos0, k, idx, out, range(T))


def test_prefill_sampled_threshold_too_high_falls_back():
    # the sampled entries (every 4th) score far above the rest, so the sampled threshold
    # admits fewer than k candidates: rows must be resolved exactly by recomputation
    log("prefill sampled threshold fallback")
    N, T, pos0, k = 100000, 8, 99000, 512
    g = torch.Generator().manual_seed(5)
    x = torch.randn(N, 128, generator=g)
    x[::4] += 0.3
    codes, scale, _ = synth.quantize_index_keys(x)
    base = synth.make_entries([N], seed=5, device=DEV)
    cache = synth.EntryCache(codes.to(DEV), scale.to(DEV), base.kv_codes, base.kv_scale,
                             base.seq_base, base.n_entries)
    q_idx = synth.bf16_bits(torch.ones(T, 128)).to(DEV)
    q = synth.make_queries(T, 5, device=DEV)
    swa = synth.make_swa(1, T + 127, 5, device=DEV)[0]
    idx, out = run_prefill(cache, q_idx, q, swa, N, 1, pos0, k)
    torch.cuda.synchronize()
    check_rows(cache, q_idx, q, swa, N, 1, pos0, k, idx, out, range(T))


def test_prefill_tied_keys_go_to_lower_entries():
    # every index key appears four times (25,000 distinct rows at random positions): a row's
    # threshold score is often shared by entries on both sides of the cut, and the row takes
    # the lowest of them (sampled threshold, candidates resolved one wave per row)
    log("prefill tied keys")
    N, T, pos0, k = 100000, 16, 99000, 512
    g = torch.Generator().manual_seed(11)
    base = torch.randn(N // 4, 128, generator=g)
    x = base[torch.randperm(N, generator=g) % (N // 4)]
    codes, scale, _ = synth.quantize_index_keys(x)
    ent = synth.make_entries([N], seed=11, device=DEV)
    cache = synth.EntryCache(codes.to(DEV), scale.to(DEV), ent.kv_codes, ent.kv_scale,
                             ent.seq_base, ent.n_entries)
    q_idx = synth.make_index_queries(T, 11, device=DEV)
    q = synth.make_queries(T, 11, device=DEV)
    swa = synth.make_swa(1, T + 127, 11, device=DEV)[0]
    idx, out = run_prefill(cache, q_idx, q, swa, N, 1, pos0, k)
    torch.cuda.synchronize()
    check_rows(cache, q_idx, q, swa, N, 1, pos0, k, idx, out, range(T))
    keys = oracle.dequant_index_keys(h(cache.idx_codes))
    kscale = h(cache.idx_scale).astype(np.float64)
    qi, gi = h(q_idx), h(idx)
    split_rows = 0
    for t in range(T):
        n_t = oracle.visible_entries(pos0 + t, 1, N)
        s = kscale[:n_t] * (keys[:n_t] @ oracle.formats.bf16_decode(qi[t]))
        order = np.lexsort((np.arange(n_t), -s))
        sk = s[order[k - 1]]
        others = np.abs(s[s != sk] - sk)
        if (s == sk).sum() > (s[order[:k]] == sk).sum() and others.min() > 1e-4 * abs(sk):
            # duplicates of the threshold score on both sides of the cut, clear of the rest
            assert np.array_equal(gi[t], np.sort(order[:k])), f"row {t}: tie not to the lower entries"
            split_rows += 1
    log(f"rows whose threshold duplicates were split: {split_rows}")
    assert split_rows >= 4


def test_prefill_rows_of_many_splits():
    # 140,000 entries: 35 entry splits, more than one wave's registers hold per row, so rows
    # are resolved a workgroup per row
    log("prefill 35 splits")
    N, T, pos0, k = 140000, 16, 139990, 512
    cache, q_idx, q, swa, idx, out = _case(N, 1, T, pos0, k, seed=13)
    check_rows(cache, q_idx, q, swa, N, 1, pos0, k, idx, out, range(T))


def test_prefill_select_and_reuse_attention_match_chunk():
    # csa2_prefill_select writes the chunk's lists; csa2_sparse_attn_prefill over them with the
    # same queries and window reproduces the chunk's output bit for bit, and a Reuse layer's
    # own queries and window over the same lists match the oracle
    log("prefill select + reuse attention")
    N, ratio, T, pos0, k = 20000, 2, 200, 39800, 512
    cache, q_idx, q, swa, idx, out = _case(N, ratio, T, pos0, k, seed=31)
    ws = csa2.prefill_workspace(T, N, k)
    idx2 = torch.empty_like(idx)
    csa2.csa2_prefill_select(q_idx, cache.idx_codes, cache.idx_scale, N, ratio, pos0, k, idx2, ws)
    out2 = torch.empty_like(out)
    aws = csa2.attn_workspace(T, k)
    csa2.csa2_sparse_attn_prefill(q, cache.kv_codes, cache.kv_scale, idx2, swa, pos0, out2, aws, SCALE)
    q_r = synth.make_queries(T, 32, device=DEV)
    swa_r = synth.make_swa(1, T + 127, 32, device=DEV)[0]
    out_r = torch.empty_like(out)
    csa2.csa2_sparse_attn_prefill(q_r, cache.kv_codes, cache.kv_scale, idx2, swa_r, pos0, out_r, aws, SCALE)
    torch.cuda.synchronize()
    assert np.array_equal(h(idx2), h(idx))
    assert np.array_equal(h(out2), h(out))
    kc, ks, g = h(cache.kv_codes), h(cache.kv_scale), h(idx2)
    for t in (0, 99, T - 1):
        p = pos0 + t
        lo = max(0, p - 127)
        win = h(swa_r)[lo - (pos0 - 127): p - (pos0 - 127) + 1]
        ref = oracle.decode_attention(h(q_r)[t], kc, ks, 0, g[t], win, win.shape[0], SCALE)
        assert attn_rel_err(h(out_r)[t], ref) <= ATTN_TOL, f"row {t}"


def test_prefill_overflow_path_all_ties():
    # every score is 0: the candidate list overflows and rows are resolved by recomputation;
    # ties go to the lowest entries
    log("prefill overflow")
    N, T, k = 20000, 8, 512
    cache, q_idx, q, swa, idx, out = _case(N, 2, T, 2 * N - T, k, seed=3, zero_q=True)
    g = h(idx)
    for t in range(T):
        assert np.array_equal(g[t], np.arange(k))
    check_rows(cache, q_idx, q, swa, N, 2, 2 * N - T, k, idx, out, [0, T - 1])


def test_prefill_matches_decode_per_row():
    # one prefill row equals a decode call over its visible entries with its window
    log("prefill vs decode")
    N, T, k, pos0 = 6000, 16, 512, 11984
    cache, q_idx, q, swa, idx, out = _case(N, 2, T, pos0, k, seed=21)
    t = T - 1
    p = pos0 + t
    n_t = (p + 1) // 2
    scores = torch.empty((1, n_t), dtype=torch.float32, device=DEV)
    csa2.csa2_index_score(q_idx[t:t + 1].contiguous(), cache.idx_codes, cache.idx_scale,
                          torch.zeros(1, dtype=torch.int64, device=DEV),
                          torch.tensor([n_t], dtype=torch.int32, device=DEV), scores)
    didx = torch.empty((1, k), dtype=torch.int32, device=DEV)
    csa2.csa2_topk(scores, torch.tensor([n_t], dtype=torch.int32, device=DEV), k, didx)
    torch.cuda.synchronize()
    # same selection rule on scores of the same precision class; compare as sets within the rule
    keys = oracle.dequant_index_keys(h(cache.idx_codes)[:n_t])
    s = h(cache.idx_scale)[:n_t].astype(np.float64) * (keys @ oracle.formats.bf16_decode(h(q_idx)[t]))
    gap = check_topk(h(didx)[0], s, k, label="decode row")
    check_topk(h(idx)[t], s, k, label="prefill row")
    if gap > 1e-4:  # a clear threshold: the two selections are the same set
        assert np.array_equal(h(didx)[0], h(idx)[t]), "prefill and decode lists differ"
    # the decode attention over the prefill row's list and its causal window equals the row
    win = swa[p - (pos0 - 127) - 127: p - (pos0 - 127) + 1][None].contiguous()
    dout = torch.empty((1, 16, 512), dtype=torch.float32, device=DEV)
    csa2.csa2_sparse_attn_decode(q[t:t + 1].contiguous(), cache.kv_codes, cache.kv_scale,
                                 torch.zeros(1, dtype=torch.int64, device=DEV), idx[t:t + 1].contiguous(),
                                 win, torch.tensor([128], dtype=torch.int32, device=DEV), dout,
                                 csa2.attn_workspace(1, k), softmax_scale=SCALE)
    torch.cuda.synchronize()
    assert attn_rel_err(h(dout)[0], h(out)[t]) <= 1e-5, "prefill and decode attention differ"


def test_c5_prefill_chunk_sampled_rows():
    cfg = synth.CONFIGS["c5_prefill"]
    T, ratio, k = cfg["T"], cfg["ratio"], cfg["k"]
    N = synth.entries_for(cfg["ctx"], ratio)
    pos0 = cfg["ctx"] - T
    log(f"c5 T={T} N={N} pos0={pos0}")
    cache, q_idx, q, swa, idx, out = _case(N, ratio, T, pos0, k, seed=cfg["seed"])
    g = h(idx)
    # properties on every row
    for t in range(T):
        n_t = (pos0 + t + 1) // ratio
        row = g[t]
        assert np.all(row >= 0) and np.all(np.diff(row) > 0) and row[-1] < n_t
    # 68 rows: both ends of the chunk, both sides of every 256-row block edge, around the
    # middle, and the rows whose visible count reaches the last multiple of 4,096 entries
    # (the contraction's entry splits), plus a seeded spread
    rows = {0, 1, 2, 3, 127, 128, 129, 2047, 2048, 2049, T - 4, T - 3, T - 2, T - 1}
    rows |= {256 * j - 1 for j in range(1, T // 256)} | {256 * j for j in range(1, T // 256)}
    rows |= {t for t in range(T) if ((pos0 + t + 1) // ratio) % 4096 in (0, 4095, 1)}
    rng = np.random.default_rng(cfg["seed"])
    rows |= set(rng.choice(T, 68 - len(rows), replace=False).tolist()) if len(rows) < 68 else set()
    rows = sorted(rows)
    assert len(rows) >= 64
    log(f"c5 oracle rows: {len(rows)}")
    check_rows(cache, q_idx, q, swa, N, ratio, pos0, k, idx, out, rows)
