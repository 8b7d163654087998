"""GPU parity of a whole 40-layer decode step (compressed_sparse_kv_csa2_amd.model) against
the oracle, at a 65,536-token context (encoder pools 32,768 entries at 1:2, decoder pool
65,536 at ratio 1, candidate pool 16,384), batch 2 with unequal window lengths.  Every
selecting layer is checked against fp64 oracle scores under the gap rule (Reindex staged
on the GPU's pool), every Reuse layer is checked to attend its source's list, and every
layer's attention against the oracle on the GPU's list.  The benchmark's full-size pass
(2^20 context) runs the same code."""
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


def test_whole_model_decode_step():
    B, n_enc, n_dec, seed = 2, 32768, 65536, 7
    log(f"model pass B={B} enc={n_enc} dec={n_dec}")
    enc = [synth.make_entries([n_enc] * B, seed=seed, device=DEV, field_base=10 * (i + 1))
           for i in range(3)]
    dec = synth.make_entries([n_dec] * B, seed=seed, device=DEV)
    q_idx = {l: synth.make_index_queries(B, seed, device=DEV, sub=l) for l in model.SELECTING}
    q = torch.stack([synth.make_queries(B, seed, device=DEV, sub=l) for l in range(40)]).contiguous()
    swa = torch.stack([synth.make_swa(B, 128, seed, device=DEV, sub=l) for l in range(40)]).contiguous()
    swa_len = torch.tensor([128, 77], dtype=torch.int32, device=DEV)
    run = model.DecodePass(B, n_enc, n_dec, device=DEV)
    run.step(enc, dec, q_idx, q, swa, swa_len)
    torch.cuda.synchronize()
    first = {l: h(t).copy() for l, t in run.lists.items()}
    out1 = h(run.out).copy()
    run.step(enc, dec, q_idx, q, swa, swa_len)  # a second step on the same buffers
    torch.cuda.synchronize()
    assert_ws_ok(*run.workspaces())
    assert all(np.array_equal(first[l], h(run.lists[l])) for l in first)
    assert np.array_equal(out1, h(run.out))

    caches = {l: enc[i] for i, l in enumerate(model.ENCODER_FULL)}
    host = {id(c): (h(c.kv_codes), h(c.kv_scale)) for c in enc + [dec]}
    pool = h(run.pool)
    for b in range(B):
        log(f"model oracle row {b}")
        for l in model.ENCODER_FULL:
            c = caches[l]
            sl = slice(b * n_enc, (b + 1) * n_enc)
            s = oracle.index_scores(h(q_idx[l])[b], h(c.idx_codes)[sl], h(c.idx_scale)[sl])
            check_topk(first[l][b], s, 512, label=f"encoder Full {l} row {b}")
        sl = slice(b * n_dec, (b + 1) * n_dec)
        codes, scale = h(dec.idx_codes)[sl], h(dec.idx_scale)[sl]
        s = oracle.index_scores(h(q_idx[20])[b], codes, scale)
        check_topk(pool[b], s, 16384, label=f"decoder pool row {b}")
        p = pool[b]
        check_topk(first[20][b], s[p], 512, ids=p, label=f"decoder own row {b}")
        for l in model.REINDEX:
            _, r = oracle.reindex_layer(h(q_idx[l])[b], codes, scale, p)
            check_topk(first[l][b], r, 512, ids=p, label=f"Reindex {l} row {b}")
        for l in range(40):
            src = None if l in model.WINDOW_ONLY else model.list_source(l)
            if src is None:
                c, base, idx = dec, b * n_dec, np.zeros(0, np.int32)
            else:
                c = dec if src >= model.DECODER_FULL else caches[src]
                base = b * (n_dec if src >= model.DECODER_FULL else n_enc)
                idx = first[src][b]
            ref = oracle.decode_attention(h(q[l])[b], *host[id(c)], base, idx,
                                          h(swa[l])[b], int(h(swa_len)[b]), SCALE)
            assert attn_rel_err(out1[l, b], ref) <= ATTN_TOL, f"layer {l} row {b}"


def test_whole_model_decode_step_full_size():
    # the benchmark's shape (2^20 context, batch 4) in its launch configuration; sampled
    # checks: sequence 3 through every selecting layer and a spread of attention layers
    B, n_enc, n_dec, seed = 4, 1 << 19, 1 << 20, 3
    log(f"model pass full size B={B} enc={n_enc} dec={n_dec}")
    enc = [synth.make_entries([n_enc] * B, seed=seed, device=DEV, field_base=10 * (i + 1))
           for i in range(3)]
    dec = synth.make_entries([n_dec] * B, seed=seed, device=DEV)
    q_idx = {l: synth.make_index_queries(B, seed, device=DEV, sub=l) for l in model.SELECTING}
    q = torch.stack([synth.make_queries(B, seed, device=DEV, sub=l) for l in range(40)]).contiguous()
    swa = torch.stack([synth.make_swa(B, 128, seed, device=DEV, sub=l) for l in range(40)]).contiguous()
    swa_len = torch.full((B,), 128, dtype=torch.int32, device=DEV)
    run = model.DecodePass(B, n_enc, n_dec, device=DEV)
    run.step(enc, dec, q_idx, q, swa, swa_len)
    torch.cuda.synchronize()
    assert_ws_ok(*run.workspaces())
    b = 3
    lists = {l: h(t)[b] for l, t in run.lists.items()}
    out = h(run.out[:, b])
    caches = {l: enc[i] for i, l in enumerate(model.ENCODER_FULL)}
    for l in model.ENCODER_FULL:
        c = caches[l]
        sl = slice(b * n_enc, (b + 1) * n_enc)
        s = oracle.index_scores(h(q_idx[l])[b], h(c.idx_codes[sl]), h(c.idx_scale[sl]))
        check_topk(lists[l], s, 512, label=f"encoder Full {l}")
    sl = slice(b * n_dec, (b + 1) * n_dec)
    codes, scale = h(dec.idx_codes[sl]), h(dec.idx_scale[sl])
    s = oracle.index_scores(h(q_idx[20])[b], codes, scale)
    p = h(run.pool)[b]
    check_topk(p, s, 16384, label="decoder pool")
    check_topk(lists[20], s[p], 512, ids=p, label="decoder own")
    for l in model.REINDEX:
        _, r = oracle.reindex_layer(h(q_idx[l])[b], codes, scale, p)
        check_topk(lists[l], r, 512, ids=p, label=f"Reindex {l}")
    for l in (0, 2, 7, 14, 19, 20, 23, 28, 39):
        src = None if l in model.WINDOW_ONLY else model.list_source(l)
        if src is None:
            c, n, idx = dec, n_dec, np.zeros(0, np.int32)
        else:
            c, n = (dec, n_dec) if src >= model.DECODER_FULL else (caches[src], n_enc)
            idx = lists[src]
        sl = slice(b * n, (b + 1) * n)
        ref = oracle.decode_attention(h(q[l])[b], h(c.kv_codes[sl]), h(c.kv_scale[sl]), 0, idx,
                                      h(swa[l])[b], 128, SCALE)
        assert attn_rel_err(out[l], ref) <= ATTN_TOL, f"layer {l}"


def test_graph_replay_equals_eager():
    """The 40-layer step captured once into a HIP graph (as the benchmark's --graph does)
    and replayed five times, with eager steps on other inputs and synchronisations between
    the replays: every replay's lists and outputs equal an eager step's on the captured
    inputs, bit for bit."""
    B, n_enc, n_dec, seed = 2, 32768, 65536, 11
    log(f"graph replay B={B} enc={n_enc} dec={n_dec}")

    def inputs(sd):
        enc = [synth.make_entries([n_enc] * B, seed=sd, device=DEV, field_base=10 * (i + 1))
               for i in range(3)]
        dec = synth.make_entries([n_dec] * B, seed=sd, device=DEV)
        q_idx = {l: synth.make_index_queries(B, sd, device=DEV, sub=l) for l in model.SELECTING}
        q = torch.stack([synth.make_queries(B, sd, device=DEV, sub=l) for l in range(40)]).contiguous()
        swa = torch.stack([synth.make_swa(B, 128, sd, device=DEV, sub=l) for l in range(40)]).contiguous()
        return enc, dec, q_idx, q, swa

    a, other = inputs(seed), inputs(seed + 1)
    swa_len = torch.tensor([128, 90], dtype=torch.int32, device=DEV)
    run = model.DecodePass(B, n_enc, n_dec, device=DEV)
    run.step(*a, swa_len)
    torch.cuda.synchronize()
    ref = [run.out.clone()] + [v.clone() for v in run.lists.values()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.step(*a, swa_len, stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(5):
        run.step(*other, swa_len)  # eager work on other inputs between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [run.out] + list(run.lists.values())
        assert all(torch.equal(x, y) for x, y in zip(ref, got)), f"replay {rep} differs from eager"
    assert_ws_ok(*run.workspaces())


def test_decode_pass_prepares_again_for_new_inputs():
    # DecodePass reuses its checked and marshalled calls while the inputs are the same
    # buffers.  A step on other buffers (new queries and windows) must give what a fresh pass
    # gives on them, and going back to the first buffers must give the first results again.
    B, n_enc, n_dec = 2, 16384, 32768
    log(f"model pass re-preparation B={B} enc={n_enc} dec={n_dec}")
    enc = [synth.make_entries([n_enc] * B, seed=5, device=DEV, field_base=10 * (i + 1)) for i in range(3)]
    dec = synth.make_entries([n_dec] * B, seed=5, device=DEV)
    swa_len = torch.tensor([128, 90], dtype=torch.int32, device=DEV)

    def inputs(seed):
        q_idx = {l: synth.make_index_queries(B, seed, device=DEV, sub=l) for l in model.SELECTING}
        q = torch.stack([synth.make_queries(B, seed, device=DEV, sub=l) for l in range(40)]).contiguous()
        swa = torch.stack([synth.make_swa(B, 128, seed, device=DEV, sub=l) for l in range(40)]).contiguous()
        return q_idx, q, swa

    a, b = inputs(11), inputs(12)
    run = model.DecodePass(B, n_enc, n_dec, device=DEV)
    run.step(enc, dec, *a, swa_len)
    torch.cuda.synchronize()
    out_a, lists_a = h(run.out).copy(), {l: h(t).copy() for l, t in run.lists.items()}
    run.step(enc, dec, *b, swa_len)
    torch.cuda.synchronize()
    fresh = model.DecodePass(B, n_enc, n_dec, device=DEV)
    fresh.step(enc, dec, *b, swa_len)
    torch.cuda.synchronize()
    assert np.array_equal(h(run.out), h(fresh.out)), "outputs on new inputs differ from a fresh pass"
    assert all(np.array_equal(h(run.lists[l]), h(fresh.lists[l])) for l in run.lists)
    assert not np.array_equal(h(run.out), out_a), "the second inputs gave the first outputs"
    run.step(enc, dec, *a, swa_len)
    torch.cuda.synchronize()
    assert np.array_equal(h(run.out), out_a)
    assert all(np.array_equal(h(run.lists[l]), lists_a[l]) for l in run.lists)
    assert_ws_ok(*run.workspaces(), *fresh.workspaces())
