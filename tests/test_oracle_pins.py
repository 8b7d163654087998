"""Pins of the CPU oracle to facts outside itself (runs without a GPU).

Each test ties an oracle function to something the oracle does not compute
itself: numbers the pages print (tests/golden/*_pages.txt), the OCP number
format tables, torch's float8 / bfloat16 casts and SDPA, exact rational
arithmetic, brute-force enumeration, closed forms and invariants.  A dropped
term, a wrong sign or index, a swapped nibble or a transposed operand in the
oracle makes at least one of them fail.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import formats
from _util import read_golden

SCALE = 1.0 / math.sqrt(512)


# --------------------------------------------------------------------------- formats
def test_e2m1_decode_matches_ocp_table():
    rows = read_golden("e2m1_ocp_mx.txt")
    codes = np.array([int(r[0]) for r in rows])
    want = np.array([float(r[1]) for r in rows])
    got = formats.e2m1_decode(codes)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))  # code 8 is -0


def test_e2m1_values_are_e4m3_exact():
    # every E2M1 value is an E4M3 value: the torch cast must reproduce it exactly
    v = torch.tensor(formats.e2m1_decode(np.arange(16)), dtype=torch.float32)
    back = v.to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(back, v.double().numpy())


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = formats.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_bf16_decode_vs_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.int64).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = formats.bf16_decode(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_unpack_order_and_scales_match_generator():
    # The generator keeps the values it meant to store; the oracle's decode of the
    # packed bytes (nibble order, E2M1, E4M3 group scales, fp32 entry scale) must
    # give them back exactly (fp32 products of a 2-bit and a <=4-bit significand).
    cache, vi, vk = synth.make_entries([37, 5], seed=11, keep_values=True)
    codes = cache.idx_codes.numpy()
    scale = cache.idx_scale.numpy()
    got_i = oracle.dequant_index_keys(codes) * scale.astype(np.float64)[:, None]
    assert np.array_equal(got_i.astype(np.float32), vi.numpy())
    got_k = oracle.dequant_main(cache.kv_codes.numpy(), cache.kv_scale.numpy())
    assert np.array_equal(got_k, vk.double().numpy())


# --------------------------------------------------------------------------- bytes & layout
def _golden_dict(name):
    return {r[0]: r[1:] for r in read_golden(name)}


def test_byte_accounting_matches_pages():
    g = _golden_dict("kv_bytes_pages.txt")
    assert oracle.main_entry_bytes() == int(g["main_entry_bytes"][0]) == \
        int(g["main_entry_values"][0]) * int(g["main_entry_value_bits"][0]) // 8 + \
        int(g["main_entry_scale_bytes"][0])
    assert oracle.index_entry_bytes() == int(g["index_entry_bytes"][0]) == \
        int(g["index_entry_values"][0]) * int(g["index_entry_value_bits"][0]) // 8 + \
        int(g["index_entry_scale_bytes"][0])
    assert oracle.main_entry_bytes() + oracle.index_entry_bytes() == int(g["entry_pair_bytes"][0])
    from oracle.csa2_ref import entries_per_token
    assert entries_per_token() == float(g["entries_per_token"][0])
    assert oracle.global_kv_bytes_per_token() == float(g["global_kv_bytes_per_token"][0])
    gib = oracle.global_kv_bytes(1 << 20) / 2 ** 30
    assert round(gib, 2) == float(g["global_kv_gib_at_1m_tokens"][0])
    # "about a quarter" of the predecessor's bytes per token
    assert 0.24 < oracle.global_kv_bytes_per_token() / float(g["v4_flash_global_kv_bytes_per_token"][0]) < 0.26


def test_layer_layout_matches_pages():
    g = _golden_dict("layer_layout_pages.txt")
    for mode in ("swa", "full", "reindex"):
        want = [int(x) for x in g[mode]]
        assert [l for l in range(40) if oracle.layer_mode(l) == mode] == want
    assert sum(oracle.layer_mode(l) == "reuse" for l in range(40)) == int(g["reuse_count"][0])
    dec = [oracle.layer_mode(l) for l in range(int(g["encoder_last"][0]) + 1, 40)]
    assert (dec.count("full"), dec.count("reindex"), dec.count("reuse")) == (1, 4, 15)
    assert [oracle.reuse_source(l) for l in (3, 7, 9, 21, 23, 25, 39)] == [2, 2, 8, 20, 20, 24, 36]


# --------------------------------------------------------------------------- scores
def _frac_bf16(bits):
    return Fraction(float(torch.tensor(int(np.int16(np.uint16(bits)))).to(torch.int16)
                          .view(torch.bfloat16).item()))


def test_index_scores_exact_against_rationals():
    table = {int(r[0]): Fraction(float(r[1])) for r in read_golden("e2m1_ocp_mx.txt")}
    cache = synth.make_entries([6], seed=5)
    q = synth.make_index_queries(1, seed=5)[0].numpy().view(np.uint16)
    codes = cache.idx_codes.numpy()
    scale = cache.idx_scale.numpy()
    got = oracle.index_scores(q, codes, scale)
    qf = [_frac_bf16(b) for b in q]
    for j in range(codes.shape[0]):
        vals = []
        for byte in codes[j]:
            vals += [table[int(byte) & 15], table[int(byte) >> 4]]
        exact = Fraction(float(scale[j])) * sum(a * b for a, b in zip(qf, vals))
        assert got[j] == float(exact)   # float(Fraction) rounds correctly to fp64
    assert oracle.index_dot_is_exact(q)


def test_index_dot_exactness_flag_detects_wide_span():
    # A query spanning ~2^-120..2^100 cannot be summed exactly in fp64.
    q = np.zeros(128, dtype=np.float32)
    q[0], q[1], q[2] = 2.0 ** 100, 2.0 ** -120, -(2.0 ** 100)
    bits = (torch.from_numpy(q).to(torch.bfloat16).view(torch.int16).numpy()).view(np.uint16)
    assert not oracle.index_dot_is_exact(bits)
    # ...because an fp64 sum of such terms depends on its order: left to right
    # loses the small term that the exact sum keeps.
    terms = oracle.formats.bf16_decode(bits) * 1.0
    seq = 0.0
    for t in terms:
        seq += t
    exact = Fraction(2) ** 100 + Fraction(2) ** -120 - Fraction(2) ** 100
    assert seq != float(exact)


# --------------------------------------------------------------------------- top-k
def _dominates(s, i, j):
    return s[i] > s[j] or (s[i] == s[j] and i < j)


@pytest.mark.parametrize("seed", range(8))
def test_topk_bruteforce_subsets(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 9))
    pool = np.array([-1.5, -0.0, 0.0, 0.5, 2.0, 2.0, 3.25])
    s = rng.choice(pool, size=n)  # forced ties, including -0 vs +0
    for k in range(0, n + 3):
        m = min(k, n)
        valid = [set(c) for c in itertools.combinations(range(n), m)
                 if all(_dominates(s, i, j) for i in c for j in range(n) if j not in c)]
        assert len(valid) == 1
        want = sorted(valid[0]) + [-1] * (k - m)
        assert list(oracle.topk(s, k)) == want


def test_topk_respects_n_valid():
    s = np.array([0.0, 1.0, 5.0, 9.0, 9.0])
    assert list(oracle.topk(s, 3, n_valid=3)) == [0, 1, 2]
    assert list(oracle.topk(s, 2, n_valid=5)) == [3, 4]
    assert list(oracle.topk(s, 4, n_valid=2)) == [0, 1, -1, -1]


def _small_entries(n, seed, dup=()):
    cache = synth.make_entries([n], seed=seed)
    codes, scale = cache.idx_codes.numpy().copy(), cache.idx_scale.numpy().copy()
    for a, b in dup:  # entry b becomes a copy of entry a (exact score ties)
        codes[b], scale[b] = codes[a], scale[a]
    return cache, codes, scale


def test_full_pool_reindex_reuse_invariants():
    n = 3000
    cache, codes, scale = _small_entries(n, 21)
    q_full = synth.make_index_queries(1, 21)[0].numpy().view(np.uint16)
    q_re = synth.make_index_queries(1, 21, sub=1)[0].numpy().view(np.uint16)
    s, pool, own = oracle.full_layer(q_full, codes, scale, n, pool_size=1024, k=64)
    assert set(own) <= set(pool)                          # own top-k inside the pool
    assert np.all(np.diff(pool) > 0) and np.all(np.diff(own) > 0)
    # pool threshold: every pooled score >= every non-pooled score
    out_mask = np.ones(n, bool); out_mask[pool] = False
    assert s[pool].min() >= s[out_mask].max()
    idx_r, s_r = oracle.reindex_layer(q_re, codes, scale, pool, k=64)
    assert set(idx_r) <= set(pool)
    full_r = oracle.index_scores(q_re, codes, scale)
    assert np.array_equal(s_r, full_r[pool])                # re-score is the same function
    assert list(idx_r) == list(oracle.topk(np.where(np.isin(np.arange(n), pool), full_r,
                                                    -np.inf), 64))
    assert np.array_equal(oracle.reuse_layer(idx_r), idx_r)


def test_reindex_ties_go_to_lowest_entry_id():
    n = 200
    cache, codes, scale = _small_entries(n, 3, dup=[(150, 40), (150, 90)])
    q = synth.make_index_queries(1, 3)[0].numpy().view(np.uint16)
    s = oracle.index_scores(q, codes, scale)
    # put the tied trio at the very top so exactly the boundary splits them
    order = np.lexsort((np.arange(n), -s))
    pool = np.sort(np.unique(np.concatenate([[40, 90, 150], order[:20]])))
    rank_of_tie = int((s[pool] > s[150]).sum())
    idx, _ = oracle.reindex_layer(q, codes, scale, pool, k=rank_of_tie + 2)
    chosen = set(idx) & {40, 90, 150}
    assert chosen == {40, 90}


# --------------------------------------------------------------------------- attention
def _sdpa(q_bits, values, scale):
    q = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).double().view(1, 16, 1, 512)
    v = torch.from_numpy(values).double().view(1, 1, -1, 512).expand(1, 16, -1, 512)
    return torch.nn.functional.scaled_dot_product_attention(q, v, v, scale=scale).view(16, 512).numpy()


def test_sparse_equals_dense_when_k_covers_all():
    n = 40
    cache, _, vk = synth.make_entries([n], seed=7, keep_values=True)
    q = synth.make_queries(1, 7)[0].numpy().view(np.uint16)
    swa = synth.make_swa(1, 128, 7)[0].numpy()
    swa_vals = torch.from_numpy(swa).view(torch.float8_e4m3fn).double().numpy()
    idx = np.arange(n, dtype=np.int32)
    got = oracle.decode_attention(q, cache.kv_codes.numpy(), cache.kv_scale.numpy(), 0, idx,
                                  swa, 100, SCALE)
    dense = _sdpa(q, np.concatenate([vk.double().numpy(), swa_vals[:100]]), SCALE)
    np.testing.assert_allclose(got, dense, rtol=1e-12, atol=1e-13)
    # order of the index list and -1 holes do not matter
    perm = np.random.default_rng(0).permutation(idx)
    holes = np.concatenate([perm, np.full(7, -1, np.int32)])
    got2 = oracle.decode_attention(q, cache.kv_codes.numpy(), cache.kv_scale.numpy(), 0, holes,
                                   swa, 100, SCALE)
    np.testing.assert_allclose(got2, got, rtol=1e-12, atol=1e-13)


def test_attention_closed_forms():
    n = 9
    cache, _, vk = synth.make_entries([n], seed=8, keep_values=True)
    vk = vk.double().numpy()
    kc, ks = cache.kv_codes.numpy(), cache.kv_scale.numpy()
    swa = synth.make_swa(1, 128, 8)[0].numpy()
    q0 = np.zeros((16, 512), np.uint16)
    out = oracle.decode_attention(q0, kc, ks, 0, np.arange(n), swa, 0, SCALE)
    np.testing.assert_allclose(out, np.broadcast_to(vk.mean(0), (16, 512)), rtol=1e-13, atol=1e-15)
    q = synth.make_queries(1, 8)[0].numpy().view(np.uint16)
    one = oracle.decode_attention(q, kc, ks, 0, np.array([4, -1, -1]), swa, 0, SCALE)
    np.testing.assert_array_equal(one, np.broadcast_to(vk[4], (16, 512)))
    empty = oracle.decode_attention(q, kc, ks, 0, np.full(5, -1), swa, 0, SCALE)
    assert np.array_equal(empty, np.zeros((16, 512)))
    swa_only = oracle.decode_attention(q, kc, ks, 0, np.full(5, -1), swa, 128, SCALE)
    swa_vals = torch.from_numpy(swa).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_allclose(swa_only, _sdpa(q, swa_vals, SCALE), rtol=1e-12, atol=1e-13)
    # a sequence offset selects the same rows as absolute indices
    sh = oracle.decode_attention(q, kc, ks, 3, np.array([1, 2]), swa, 0, SCALE)
    np.testing.assert_allclose(sh, _sdpa(q, vk[[4, 5]], SCALE), rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------- prefill
def test_prefill_visible_counts_closed_form():
    pos0, T, ratio, N = 262144 - 4096, 4096, 2, 131072
    counts = [oracle.visible_entries(pos0 + t, ratio, N) for t in range(T)]
    assert counts[0] == 129024 and counts[-1] == 131072
    assert sum(counts) == 2048 * (258049 + 2047) == 532_676_608
    assert oracle.visible_entries(0, 2, 10) == 0 and oracle.visible_entries(1, 2, 10) == 1
    assert oracle.visible_entries(5, 1, 3) == 3


def test_prefill_rows_equal_decode_and_ignore_future_entries():
    N, ratio, T, k = 300, 2, 40, 16
    pos0 = 2 * N - T  # chunk at the tail of the context
    cache = synth.make_entries([N], seed=9)
    qi = synth.make_index_queries(T, 9).numpy().view(np.uint16)
    q = synth.make_queries(T, 9).numpy().view(np.uint16)
    swa = synth.make_swa(1, T + 127, 9)[0].numpy()
    ic, isc = cache.idx_codes.numpy(), cache.idx_scale.numpy()
    kc, ks = cache.kv_codes.numpy(), cache.kv_scale.numpy()
    idx, out = oracle.prefill_chunk(qi, q, ic, isc, kc, ks, N, ratio, pos0, k, swa, SCALE,
                                    rows=[0, 17, T - 1])
    for t in (0, 17, T - 1):
        p = pos0 + t
        n_t = (p + 1) // ratio
        want_idx = oracle.topk(oracle.index_scores(qi[t], ic[:n_t], isc[:n_t]), k)
        assert np.array_equal(idx[t], want_idx)
        win = swa[t: t + 128]
        want = oracle.decode_attention(q[t], kc, ks, 0, want_idx, win, 128, SCALE)
        np.testing.assert_array_equal(out[t], want)
    # entries after the visible prefix cannot change row 0
    ic2, isc2, kc2 = ic.copy(), isc.copy(), kc.copy()
    n0 = (pos0 + 1) // ratio
    ic2[n0:] ^= 0x77; isc2[n0:] *= 3; kc2[n0:] ^= 0x55
    idx2, out2 = oracle.prefill_chunk(qi, q, ic2, isc2, kc2, ks, N, ratio, pos0, k, swa, SCALE,
                                      rows=[0])
    assert np.array_equal(idx2[0], idx[0]) and np.array_equal(out2[0], out[0])


def test_prefill_window_clipped_at_sequence_start():
    N, ratio, T, k = 8, 2, 6, 4
    cache = synth.make_entries([N], seed=10)
    qi = synth.make_index_queries(T, 10).numpy().view(np.uint16)
    q = synth.make_queries(T, 10).numpy().view(np.uint16)
    swa = synth.make_swa(1, T + 127, 10)[0].numpy()
    args = (cache.idx_codes.numpy(), cache.idx_scale.numpy(), cache.kv_codes.numpy(),
            cache.kv_scale.numpy())
    idx, out = oracle.prefill_chunk(qi, q, *args, N, ratio, 0, k, swa, SCALE)
    assert list(idx[0]) == [-1] * 4                 # position 0 sees no full entry at 1:2
    assert list(idx[3]) == [0, 1, -1, -1]           # position 3 sees entries 0 and 1
    swa_vals = torch.from_numpy(swa).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_allclose(out[0], _sdpa(q[0], swa_vals[127:128], SCALE), rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------- chain
def test_decoder_chain_shares_lists():
    n = 2048
    cache = synth.make_entries([n], seed=12)
    qi = {l: synth.make_index_queries(1, 12, sub=l)[0].numpy().view(np.uint16) for l in range(20, 40)}
    q = {l: synth.make_queries(1, 12, sub=l)[0].numpy().view(np.uint16) for l in range(20, 40)}
    sw = {l: synth.make_swa(1, 128, 12, sub=l)[0].numpy() for l in range(20, 40)}
    res, pool = oracle.decoder_chain(qi, q, sw, 128, cache.idx_codes.numpy(), cache.idx_scale.numpy(),
                                     cache.kv_codes.numpy(), cache.kv_scale.numpy(), 0, n,
                                     pool_size=256, k=32)
    for l in range(20, 40):
        src = oracle.reuse_source(l)
        assert np.array_equal(res[l][0], res[src][0])
        if oracle.layer_mode(l) == "reindex":
            assert set(res[l][0]) <= set(pool)
    # Reuse layers differ only through their own query and window
    assert not np.allclose(res[21][1], res[22][1])


# --------------------------------------------------------------------------- compositions
# Constructed inputs whose selections and outputs are known by construction, so the
# compositions decode_step_long and decoder_chain are pinned to closed forms, not to the
# oracle's own component functions.  Indexer entry j carries its Full-query score in
# dimension 0 and a Reindex score per Reindex layer in dimensions 1..4; a query that is
# one-hot on dimension d therefore scores entry j as scale_j * e2m1(code_jd).  Main entry
# j is the constant vector v_j * ones(512) (all codes equal, every E4M3 scale 1.0), and
# window row t of layer l is the constant w_l * ones(512).  With q_h = a * ones(512) a
# head's logits are a * sqrt(512) * (entry value), so each output row is the constant
# softmax-weighted mean of the attended values: a one-dimensional closed form.
_E2M1_CODE = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}
_E4M3_ONE = 0x38       # 1.0 in E4M3 (exponent 7, mantissa 0)
_E4M3_CODE = {0.5: 0x30, 1.0: 0x38, 2.0: 0x40, 3.0: 0x44, 4.0: 0x48}


def _bf16_bits(x):
    b = np.asarray(x, dtype=np.float32).view(np.uint32) >> 16
    assert np.array_equal((b << 16).view(np.float32), np.asarray(x, dtype=np.float32))
    return b.astype(np.uint16)


def _onehot_query(d):
    v = np.zeros(128, dtype=np.float32)
    v[d] = 1.0
    return _bf16_bits(v)


def _const_query(a):
    return _bf16_bits(np.full((16, 512), a, dtype=np.float32))


def _pack_index_entries(dims):
    """dims: [n][5] E2M1 values of dimensions 0..4 (the rest 0) -> codes u8 [n][64]."""
    n = len(dims)
    nib = np.zeros((n, 128), dtype=np.uint8)
    for j, row in enumerate(dims):
        for d, v in enumerate(row):
            nib[j, d] = _E2M1_CODE[float(v)]
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def _pack_main_entries(vals):
    """vals[j]: E2M1 value of every one of entry j's 512 elements (scale 1.0)."""
    n = len(vals)
    codes = np.zeros((n, 256), dtype=np.uint8)
    for j, v in enumerate(vals):
        c = _E2M1_CODE[float(v)]
        codes[j, :] = c | (c << 4)
    return codes, np.full((n, 32), _E4M3_ONE, dtype=np.uint8)


def _weighted_mean(values, a):
    """Closed form of one output element when every attended row is c * ones(512)."""
    v = np.asarray(values, dtype=np.float64)
    z = a * math.sqrt(512.0) * v  # (q . v) / sqrt(512) with q = a * ones
    w = np.exp(z - z.max())
    return float((w * v).sum() / w.sum())


def _chain_fixture(n_before=9, n=40, n_after=7, pool=12, k=3):
    """A sequence of n entries at seq_base = n_before inside a buffer with n_before entries
    in front and n_after behind (all of which score highest for every query: a wrong slice
    selects them).  Construction, by the entry's local index j:
      Full score  (dim 0):  pool members P = {2, 5, ..., 35} (12 entries, every third from 2)
                            score 4 or 6; the Full layer's own top-k F = {5, 20, 35} score
                            6 * scale, the rest of P 4 * scale; everything else 0.5 * scale.
      Reindex score of layer r (dim 1 + r): inside P the layer's own set R_r (3 entries,
                            disjoint from F and from the other layers' sets) scores 6, the
                            rest of P 1; OUTSIDE P every entry scores 6 * 2 (scale 2), so a
                            Reindex that searched beyond the pool picks them instead.
    Main values: F entries 2.0, R_r entries 3.0 + r (as E2M1: 3, 4, 6, 6), others 0.5."""
    P = list(range(2, 2 + 3 * pool, 3))
    F = [5, 20, 35]
    R = [[2, 8, 11], [14, 17, 23], [26, 29, 32]]
    dims, scale, main = [], [], []
    total = n_before + n + n_after
    for g in range(total):
        j = g - n_before
        if j < 0 or j >= n:          # outside the sequence: top score for every query
            dims.append([6.0] * 5)
            scale.append(4.0)
            main.append(0.5)
            continue
        row = [0.5, 1.0, 1.0, 1.0, 1.0]
        sc = 1.0
        if j in P:
            row[0] = 6.0 if j in F else 4.0
            for r, Rr in enumerate(R):
                row[1 + r] = 6.0 if j in Rr else 1.0
        else:
            sc = 2.0                  # off-pool entries: Reindex score 12 > 6 (and Full 1.0)
            row = [0.5, 6.0, 6.0, 6.0, 6.0]
        dims.append(row)
        scale.append(sc)
        main.append(2.0 if j in F else next((3.0 + r if r < 2 else 6.0 for r, Rr in enumerate(R)
                                             if j in Rr), 0.5))
    codes = _pack_index_entries(dims)
    kvc, kvs = _pack_main_entries(main)
    fx = dict(codes=codes, scale=np.asarray(scale, np.float32), kvc=kvc, kvs=kvs,
              base=n_before, n=n, P=P, F=F, R=R, pool=pool, k=k,
              value=lambda j: main[n_before + j])
    # with these scales the Full scores of P are 6 or 4 (x1), off-pool 0.5 x 2 = 1: P is the
    # top-12; off-pool Reindex scores 6 x 2 = 12 beat every pool entry's 6 or 1
    return fx


def _swa_const(w, length=128):
    return np.full((length, 512), _E4M3_CODE[w], dtype=np.uint8)


def test_decode_step_long_constructed():
    fx = _chain_fixture()
    a = 2.0 ** -5
    swa_len = 5
    pool, idx, out = oracle.decode_step_long(
        _onehot_query(0), _onehot_query(2), _const_query(a), fx["codes"], fx["scale"], fx["kvc"],
        fx["kvs"], fx["base"], fx["n"], _swa_const(0.5), swa_len, pool_size=fx["pool"],
        k=fx["k"])
    assert list(pool) == fx["P"]                    # local ids of the pool, ascending
    assert list(idx) == fx["R"][1]                  # Reindex layer 1's set, inside the pool
    want = _weighted_mean([fx["value"](j) for j in fx["R"][1]] + [0.5] * swa_len, a)
    np.testing.assert_allclose(out, np.full((16, 512), want), rtol=1e-12)
    # the window rows beyond swa_len are never attended
    _, _, out2 = oracle.decode_step_long(
        _onehot_query(0), _onehot_query(2), _const_query(a), fx["codes"], fx["scale"], fx["kvc"],
        fx["kvs"], fx["base"], fx["n"], np.concatenate([_swa_const(0.5, swa_len),
                                                        _swa_const(4.0, 128 - swa_len)]),
        swa_len, pool_size=fx["pool"], k=fx["k"])
    np.testing.assert_array_equal(out2, out)


def test_decoder_chain_constructed():
    fx = _chain_fixture()
    layers = range(20, 32)          # Full 20, Reuse 21-23, Reindex 24, Reuse 25-27, Reindex 28 ...
    # the Full layer uses dim 0; Reindex layers 24, 28 use dims 1, 2 (sets R[0], R[1])
    qi = {l: _onehot_query(0) for l in layers}
    qi[24], qi[28] = _onehot_query(1), _onehot_query(2)
    wvals = [0.5, 1.0, 2.0, 3.0, 4.0]
    a_of = {l: 2.0 ** -(4 + (l % 3)) for l in layers}
    w_of = {l: wvals[l % 5] for l in layers}
    q = {l: _const_query(a_of[l]) for l in layers}
    sw = {l: _swa_const(w_of[l]) for l in layers}
    swa_len = 7
    res, pool = oracle.decoder_chain(qi, q, sw, swa_len, fx["codes"], fx["scale"], fx["kvc"],
                                     fx["kvs"], fx["base"], fx["n"], pool_size=fx["pool"],
                                     k=fx["k"], first=20, last=31)
    assert list(pool) == fx["P"]
    want_list = {}
    for l in layers:
        want_list[l] = fx["F"] if l < 24 else fx["R"][0] if l < 28 else fx["R"][1]
        assert list(res[l][0]) == want_list[l], l
        want = _weighted_mean([fx["value"](j) for j in want_list[l]] + [w_of[l]] * swa_len, a_of[l])
        np.testing.assert_allclose(res[l][1], np.full((16, 512), want), rtol=1e-12, err_msg=str(l))
    # swapping two layers' queries and windows swaps their outputs (and nothing else moves)
    q2, sw2 = dict(q), dict(sw)
    q2[21], q2[26] = q[26], q[21]
    sw2[21], sw2[26] = sw[26], sw[21]
    res2, _ = oracle.decoder_chain(qi, q2, sw2, swa_len, fx["codes"], fx["scale"], fx["kvc"],
                                   fx["kvs"], fx["base"], fx["n"], pool_size=fx["pool"], k=fx["k"],
                                   first=20, last=31)
    got21 = _weighted_mean([fx["value"](j) for j in want_list[21]] + [w_of[26]] * swa_len, a_of[26])
    np.testing.assert_allclose(res2[21][1], np.full((16, 512), got21), rtol=1e-12)
    for l in layers:
        if l not in (21, 26):
            np.testing.assert_array_equal(res2[l][1], res[l][1])
