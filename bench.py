"""Throughput of the CSA2 path on one MI355X, with its roofline and the CPU oracle beside it.

Default workload (the one the headline line is quoted on), the decoder step at a 2^20-token
context for a batch of 4 sequences:
  Full scan of 1,048,576 FP4 indexer keys per sequence (csa2_index_score, fused level-1
  radix histogram) -> candidate pool of 16,384 (csa2_topk) -> Reindex re-score of the pool
  with the next layer's indexer query (csa2_index_score over the pool) -> its top-512
  (csa2_topk) -> gather-dequant attention of 16 heads x 512 merged with a 128-row FP8
  window (csa2_sparse_attn_decode).
Layer modes and pool: "DeepSeek-V4.1 模型结构（0）：一张图看懂 DeepSeek-V4.1-Flash", commentary
on the four layer modes; "从V4到V4.1 Flash：架构的激进进化", decoder section (a first full scan
builds a pool of about 16K positions; later layers pick their top-512 inside it).

Other workloads (--workload): c2 = 32 sequences x 32,768 entries, Full decode; c3 = the
20-layer decoder chain (1 Full + 4 Reindex + 15 Reuse) at 131,072 entries x 16 sequences;
c5 = a 4,096-query prefill chunk against 131,072 entries (causal BF16 MFMA indexer, per-query
top-512, attention).

Inputs are seeded synthetic N(0,1) values quantised to the entry formats (synth.py), already
resident in HBM when timing starts.  Independent input sets are rotated step by step so the
caches never hold the bytes a step reads (a decode set's indexer keys are larger than the
256 MiB last-level cache, or enough sets are kept to exceed it).

Prints ONE JSON line.  `roofline` is for the dominant kernel: its algorithmic bytes (or
flops) per launch divided by its average launch time, measured with events on the launch
stream inside the timed region.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "CSA2 decode query-tokens/s at 2^20 ctx; achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense BF16 MFMA, published
IDX_ENTRY_BYTES = 68         # 128 x 4 bit + 4-byte scale
MAIN_ENTRY_BYTES = 288       # 512 x 4 bit + 32 E4M3 scale bytes
D_KV, HEADS, SWA, D_IDX = 512, 16, 128, 128
SCAN_SOURCES = tuple("compressed_sparse_kv_csa2_amd/csrc/" + f for f in
                     ("fsel.hip", "index_topk.hip", "scan_device.h", "select_device.h",
                      "csa2_device.h", "csa2_internal.h"))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_fseg_k_fpick_c4_long_decode_traffic.md")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-per-layer", action="store_true",
                   help="c4: leave out the per-layer path's timing (for counter runs of the chained call)")
    p.add_argument("--workload", default="c4", choices=["c4", "c2", "c3", "c5", "c5r4", "append", "model", "replay"])
    p.add_argument("--sets", type=int, default=0, help="input sets rotated per step (0: the "
                   "workload's default)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--select", default="chain", choices=["chain", "fused", "unfused"],
                   help="decode selections: csa2_select_chain (one launch), csa2_index_topk per "
                        "layer, or csa2_index_score + csa2_topk per layer")
    p.add_argument("--cpu-rows", type=int, default=0,
                   help="queries of the first input set the CPU oracle runs (0: default)")
    p.add_argument("--graph", action="store_true",
                   help="model workload: capture the 40-layer step into a HIP graph and replay it")
    p.add_argument("--no-phases", action="store_true",
                   help="skip the separate, untimed per-phase timing pass")
    p.add_argument("--read-probe", type=int, default=0, metavar="MIB",
                   help="instead of a workload, time a plain streaming read (a float32 sum) of "
                        "MIB MiB, the practical HBM read ceiling the scan is compared with")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="instead of a workload, run 5 plain device copies of MIB MiB (the "
                        "known-size reference for scaling the HBM counters) and exit")
    return p.parse_args()


def copy_calibration(mib):
    """Five device-to-device copies of `mib` MiB: a kernel of known traffic (mib MiB read and
    mib MiB written per dispatch) against which rocprofv3's FETCH_SIZE / WRITE_SIZE are scaled."""
    import torch
    n = mib << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    print(json.dumps({"copy_calibration_bytes_per_dispatch": n, "dispatches": 5}), flush=True)


def read_probe(mib):
    """A plain streaming read: torch's float32 sum over `mib` MiB, 20 timed repetitions."""
    import torch
    x = torch.ones((mib << 20) // 4, dtype=torch.float32, device="cuda:0")
    for _ in range(3):
        x.sum()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(20):
        r = x.sum()
    ev[1].record()
    torch.cuda.synchronize()
    assert float(r.item()) == float(x.numel())
    us = ev[0].elapsed_time(ev[1]) * 1e3 / 20
    print(json.dumps({"read_probe_bytes": x.numel() * 4, "avg_us": round(us, 2),
                      "read_gbs": round(x.numel() * 4 / (us * 1e-6) / 1e9, 1)}), flush=True)


def cpu_info():
    """Logical CPUs of the host and its model name (from /proc/cpuinfo when present)."""
    model = None
    try:
        for line in open("/proc/cpuinfo", encoding="utf-8"):
            if line.lower().startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return os.cpu_count(), model


def timed_oracle(fn, threads):
    """Runs fn() with the BLAS pool limited to `threads` (None: as configured); seconds."""
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # threadpoolctl missing: no limit can be set
        threadpool_limits = None
    t0 = time.perf_counter()
    if threads is not None and threadpool_limits is not None:
        with threadpool_limits(limits=threads, user_api="blas"):
            fn()
    else:
        fn()
    return time.perf_counter() - t0


def scan_source_digest() -> str:
    h = hashlib.sha256()
    for rel in SCAN_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch of the fused Full scan + top-k from the committed rocprofv3 counter
    summary, or None when the summary is absent or was taken on other kernel sources."""
    try:
        text = open(TRAFFIC_FILE, encoding="utf-8").read()
    except OSError:
        return None
    m_src = re.search(r"source_digest:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_b or m_src.group(1) != scan_source_digest():
        return None
    return float(m_b.group(1))


def host(t):
    import numpy as np
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()
                    if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: numpy's BLAS pool size unknown
        return 1


class _NullEvent:
    def record(self, stream=None):
        pass


_NULL = _NullEvent()


class Marks:
    """Phase-boundary events of one step; unset slots record nothing."""

    def __init__(self, events):
        self.events = events

    def __getitem__(self, j):
        e = self.events[j]
        return e if e is not None else _NULL


# ------------------------------------------------------------------------------------ decode
class DecodeSet:
    """One input set: B sequences x N entries, plus per-layer queries and windows."""

    def __init__(self, synth, torch, B, N, seed, dev, layers):
        self.cache = synth.make_entries([N] * B, seed=seed, device=dev)
        self.q_idx = {l: synth.make_index_queries(B, seed, device=dev, sub=l) for l in layers}
        self.q = {l: synth.make_queries(B, seed, device=dev, sub=l) for l in layers}
        self.swa = {l: synth.make_swa(B, SWA, seed, device=dev, sub=l) for l in layers}
        self.swa_len = torch.full((B,), SWA, dtype=torch.int32, device=dev)


class Decode:
    """Decode workloads: c4 (2^20, pool + one Reindex), c2 (Full, no pool), c3 (decoder chain)."""

    REINDEX = (24, 28, 32, 36)

    def __init__(self, name, args, torch, synth, csa2, dev):
        self.name, self.torch, self.csa2, self.dev = name, torch, csa2, dev
        key = {"c4": "c4_long_decode", "c2": "c2_batched_full", "c3": "c3_decoder_chain"}[name]
        self.cfg = cfg = synth.CONFIGS[key]
        self.B, self.N = cfg["B"], cfg["ctx"] // cfg["ratio"]
        self.K, self.POOL = cfg["k"], cfg["pool"]
        self.layers = {"c3": list(range(20, 40)), "c4": [20, 24], "c2": [2]}[name]
        n_sets = args.sets or {"c4": 4, "c2": 8, "c3": 2}[name]
        print(f"generating {n_sets} input sets of {self.B} x {self.N} entries", file=sys.stderr,
              flush=True)
        self.sets = [DecodeSet(synth, torch, self.B, self.N, cfg["seed"] + 1000 * s, dev, self.layers)
                     for s in range(n_sets)]
        B, N = self.B, self.N
        self.mode = args.select
        if self.mode == "unfused":  # csa2_index_score + csa2_topk, the scores written out
            self.ws = [csa2.topk_workspace(B, N, self.POOL or self.K, device=dev) for _ in self.sets]
            self.scores = torch.empty((B, N), dtype=torch.float32, device=dev)
        elif self.mode == "fused" or not self.POOL:  # csa2_index_topk per selection
            self.fws = csa2.index_topk_workspace(B, N, self.POOL or self.K, device=dev)
            if self.POOL:
                self.rws = csa2.index_topk_workspace(B, self.POOL, self.K, device=dev)
        else:                       # csa2_select_chain: every selection in one launch
            self.cws = csa2.select_chain_workspace(B, N, self.POOL, device=dev)
            re = [l for l in self.layers[1:] if l in self.REINDEX]
            self.re_layers = re
            self.re_out = torch.empty((len(re), B, self.K), dtype=torch.int32, device=dev)
            for s_ in self.sets:
                s_.q_re = torch.stack([s_.q_idx[l] for l in re]).contiguous()
        if self.POOL:
            self.pool = torch.empty((B, self.POOL), dtype=torch.int32, device=dev)
            self.pool_scores = torch.empty((B, self.POOL), dtype=torch.float32, device=dev)
            self.rescore = torch.empty((B, self.POOL), dtype=torch.float32, device=dev)
            self.pool_valid = torch.full((B,), self.POOL, dtype=torch.int32, device=dev)
        self.idx = {l: torch.empty((B, self.K), dtype=torch.int32, device=dev) for l in self.layers}
        self.out = {l: torch.empty((B, HEADS, D_KV), dtype=torch.float32, device=dev)
                    for l in self.layers}
        self.attn_ws = csa2.attn_workspace(B, self.K, device=dev)
        self.stream = torch.cuda.current_stream()
        self.queries_per_step = B
        self.n_marks = 4
        self.phase_names = (["select_chain_us", None, "attention_us"]
                            if self.mode == "chain" and self.POOL else
                            ["full_scan_select_us", "reindex_select_us", "attention_us"])

    def step(self, i, marks=None):
        """One pass of the whole path over input set i % n.  marks[j] (events) are recorded at
        the phase boundaries: 0 before the Full layer, 1 after its scan and selection, 2 before
        the attentions, 3 at the end."""
        csa2, s = self.csa2, self.stream
        w = self.sets[i % len(self.sets)]
        c = w.cache
        m = marks if marks is not None else Marks([None] * 4)
        first = self.layers[0]
        full_k = self.POOL or self.K
        full_out = self.pool if self.POOL else self.idx[first]
        full_scores = self.pool_scores if self.name == "c3" else None
        m[0].record(s)
        lists = {}
        if self.mode == "chain" and self.POOL:
            own = self.idx[first] if self.name == "c3" else None
            csa2.csa2_select_chain(w.q_idx[first], c.idx_codes, c.idx_scale, c.seq_base, c.n_entries,
                                   self.N, self.pool, self.cws, k=self.K, own_out=own,
                                   q_re=w.q_re, re_out=self.re_out, stream=s)
            m[1].record(s)
            if own is not None:
                lists[first] = own
            for j, l in enumerate(self.re_layers):
                lists[l] = self.re_out[j]
            for l in self.layers[1:]:
                if l not in lists:  # Reuse: the list of the most recent Full/Reindex layer
                    lists[l] = lists[max(x for x in lists if x <= l)]
        else:
            if self.mode == "unfused":
                tw = self.ws[i % len(self.sets)]
                csa2.csa2_index_score(w.q_idx[first], c.idx_codes, c.idx_scale, c.seq_base,
                                      c.n_entries, self.scores, topk_ws=tw, stream=s)
                csa2.csa2_topk(self.scores, c.n_entries, full_k, full_out, score_out=full_scores,
                               hist_fused=True, workspace=tw, stream=s)
            else:
                csa2.csa2_index_topk(w.q_idx[first], c.idx_codes, c.idx_scale, c.seq_base,
                                     c.n_entries, full_k, full_out, self.fws, self.N,
                                     score_out=full_scores, stream=s)
            m[1].record(s)
            if self.name == "c2":
                lists[first] = self.idx[first]
            else:
                if self.name == "c3":  # the Full layer's own top-512, inside its pool
                    csa2.csa2_topk(self.pool_scores, self.pool_valid, self.K, self.idx[first],
                                   cand=self.pool, stream=s)
                    lists[first] = self.idx[first]
                for l in self.layers[1:]:
                    if l in self.REINDEX:
                        if self.mode == "unfused":
                            csa2.csa2_index_score(w.q_idx[l], c.idx_codes, c.idx_scale, c.seq_base,
                                                  self.pool_valid, self.rescore, cand=self.pool,
                                                  topk_ws=tw, stream=s)
                            csa2.csa2_topk(self.rescore, self.pool_valid, self.K, self.idx[l],
                                           cand=self.pool, hist_fused=True, workspace=tw, stream=s)
                        else:
                            csa2.csa2_index_topk(w.q_idx[l], c.idx_codes, c.idx_scale, c.seq_base,
                                                 self.pool_valid, self.K, self.idx[l], self.rws,
                                                 self.POOL, cand=self.pool, stream=s)
                        lists[l] = self.idx[l]
                    else:  # Reuse: the list of the most recent Full/Reindex layer
                        lists[l] = lists[max(x for x in lists if x <= l)]
        m[2].record(s)
        att_layers = self.layers if self.name == "c3" else [self.layers[-1]]
        for l in att_layers:
            csa2.csa2_sparse_attn_decode(w.q[l], c.kv_codes, c.kv_scale, c.seq_base, lists[l],
                                         w.swa[l], w.swa_len, self.out[l], self.attn_ws, stream=s)
        m[3].record(s)
        self.last_lists, self.last_out = lists, [self.out[l] for l in att_layers]

    def dominant(self):
        sel = "pool, own and Reindex top-512s" if self.name == "c3" else "pool and Reindex top-512"
        kernel = {"unfused": "Full scan + top-k as separate launches (k_index_score, k_topk_*)",
                  "fused": "csa2_index_topk: k_fseg<false> (segment scans and cuts) + k_fpick<false> "
                           "(exact top-k); the call timed",
                  "chain": f"csa2_select_chain: k_fseg<false> (segment scans and cuts, Reindex "
                           f"re-scores) + k_fpick<false> ({sel}); the call timed"
                  }[self.mode if self.POOL else "fused"]
        return {"kernel": kernel, "bound": "hbm", "unit": "GB/s",
                "peak": HBM_PEAK_GBS, "work": self.B * self.N * IDX_ENTRY_BYTES,
                "scale": 1e9, "marks": (0, 1)}

    def step_bytes(self):
        """Algorithmic bytes of one step: every scanned key, the pool ids, every re-scored pool
        entry with its id, each attention's gathered entries with their ids, window, q, out."""
        B, N, K = self.B, self.N, self.K
        n_att = 20 if self.name == "c3" else 1
        n_re = {"c3": 4, "c4": 1, "c2": 0}[self.name]
        per_q = N * IDX_ENTRY_BYTES + D_IDX * 2 * (1 + n_re)
        if self.POOL:
            per_q += self.POOL * 4 + n_re * self.POOL * (IDX_ENTRY_BYTES + 4)
        per_q += n_att * (K * (MAIN_ENTRY_BYTES + 4) + SWA * D_KV + HEADS * D_KV * 2 + HEADS * D_KV * 4)
        return B * per_q

    def workspaces(self):
        """The selection workspaces that start with a status block (not the two-launch top-k's)."""
        return [w for w in (getattr(self, "cws", None), getattr(self, "fws", None),
                            getattr(self, "rws", None)) if w is not None]

    def valid(self):
        """Every list strictly ascending and non-negative, every output finite, and every
        selection workspace's status block free of error bits."""
        ok = True
        for lst in self.last_lists.values():
            ok &= bool(((lst[:, 1:] > lst[:, :-1]).all() & (lst >= 0).all()).item())
        for o in self.last_out:
            ok &= bool(self.torch.isfinite(o).all().item())
        self.status = [self.csa2.csa2_workspace_status(w) for w in self.workspaces()]
        ok &= all(bits == 0 for bits, _ in self.status)
        return ok

    def per_layer(self, steps):
        """c4 as a decoder runs it layer by layer: the Full layer's scan and pool
        (csa2_index_topk), then the Reindex layer's own call on that pool with its own query
        (csa2_index_topk over the pool), then its attention.  Returns the timing, the
        phases, and whether the lists equal the chained call's."""
        torch, csa2, B, s = self.torch, self.csa2, self.B, self.stream
        fws = csa2.index_topk_workspace(B, self.N, self.POOL, device=self.dev)
        rws = csa2.index_topk_workspace(B, self.POOL, self.K, device=self.dev)
        pool = torch.empty((B, self.POOL), dtype=torch.int32, device=self.dev)
        idx = torch.empty((B, self.K), dtype=torch.int32, device=self.dev)
        out = torch.empty((B, HEADS, D_KV), dtype=torch.float32, device=self.dev)
        full, re = self.layers[0], self.re_layers[0]

        def step(i, ev=None):
            w = self.sets[i % len(self.sets)]
            c = w.cache
            if ev: ev[0].record(s)
            csa2.csa2_index_topk(w.q_idx[full], c.idx_codes, c.idx_scale, c.seq_base, c.n_entries,
                                 self.POOL, pool, fws, self.N, stream=s)
            if ev: ev[1].record(s)
            csa2.csa2_index_topk(w.q_idx[re], c.idx_codes, c.idx_scale, c.seq_base, self.pool_valid,
                                 self.K, idx, rws, self.POOL, cand=pool, stream=s)
            if ev: ev[2].record(s)
            csa2.csa2_sparse_attn_decode(w.q[re], c.kv_codes, c.kv_scale, c.seq_base, idx, w.swa[re],
                                         w.swa_len, out, self.attn_ws, stream=s)
            if ev: ev[3].record(s)

        for i in range(5):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        reps = max(20, min(100, steps))
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
        for i in range(reps):
            step(i, evs[i])
        torch.cuda.synchronize()
        ph = [round(sum(e[j].elapsed_time(e[j + 1]) for e in evs) * 1e3 / reps, 2) for j in range(3)]
        # the same input set through both paths: the Reindex list must be the chain's
        self.step(0)
        step(0)
        torch.cuda.synchronize()
        same = bool(torch.equal(idx, self.re_out[0]))
        st = [csa2.csa2_workspace_status(w) for w in (fws, rws)]
        ok = same and all(bits == 0 for bits, _ in st) and \
            bool(((idx[:, 1:] > idx[:, :-1]).all() & (idx >= 0).all()).item()) and \
            bool(torch.isfinite(out).all().item())
        return {"ms_per_step": round(ms, 5), "value": round(B / (ms * 1e-3), 1),
                "phases_us": {"full_scan_pool_us": ph[0], "reindex_select_us": ph[1],
                              "attention_us": ph[2]},
                "reindex_equals_chain": same, "valid": ok,
                "calls": "csa2_index_topk (pool) -> csa2_index_topk over the pool (Reindex) -> "
                         "csa2_sparse_attn_decode"}

    def config(self, n_sets):
        desc = {"c4": "c4_long_decode: decoder step at 2^20 ctx, batch 4, Full scan of 1,048,576 "
                      "entries -> pool 16,384 -> Reindex top-512 -> attention 16x512 + SWA 128",
                "c2": "c2_batched_full: Full decode, batch 32 x 32,768 entries (65,536-token ctx at "
                      "1:2), top-512, attention 16x512 + SWA 128",
                "c3": "c3_decoder_chain: 20 decoder layers (1 Full + 4 Reindex + 15 Reuse), batch "
                      "16 x 131,072 entries, pool 16,384, top-512, 20 attentions 16x512 + SWA 128"}
        return {"workload": desc[self.name], "batch": self.B, "context_tokens": self.cfg["ctx"],
                "entries": self.N, "pool": self.POOL, "top_k": self.K, "heads": HEADS,
                "head_dim": D_KV, "swa": SWA, "input_sets_rotated": n_sets}

    def cpu_baseline(self, rows):
        """The fp64 oracle on the host: the same step for `rows` sequences of the first set."""
        import oracle
        w, B, N = self.sets[0], self.B, self.N
        rows = max(1, min(rows or {"c4": 4, "c2": 32, "c3": 4}[self.name], B))
        c = w.cache
        codes, scale = host(c.idx_codes[: rows * N]), host(c.idx_scale[: rows * N])
        kvc, kvs = host(c.kv_codes[: rows * N]), host(c.kv_scale[: rows * N])
        qi = {l: host(v) for l, v in w.q_idx.items()}
        q = {l: host(v) for l, v in w.q.items()}
        sw = {l: host(v) for l, v in w.swa.items()}
        def one(b):
            base = b * N
            if self.name == "c4":
                oracle.decode_step_long(qi[20][b], qi[24][b], q[24][b], codes, scale, kvc, kvs, base,
                                        N, sw[24][b], SWA, self.POOL, self.K)
            elif self.name == "c2":
                _, _, own = oracle.full_layer(qi[2][b], codes[base:base + N], scale[base:base + N],
                                              N, None, self.K)
                oracle.decode_attention(q[2][b], kvc, kvs, base, own, sw[2][b], SWA)
            else:
                oracle.decoder_chain({l: v[b] for l, v in qi.items()}, {l: v[b] for l, v in q.items()},
                                     {l: v[b] for l, v in sw.items()}, SWA, codes, scale, kvc, kvs,
                                     base, N, self.POOL, self.K)

        dt = timed_oracle(lambda: [one(b) for b in range(rows)], None)
        dt1 = timed_oracle(lambda: one(0), 1)
        what = {"c4": "full 1,048,576-entry scan, pool, Reindex, attention each",
                "c2": "full 32,768-entry scan, top-512, attention each",
                "c3": "the 20-layer chain over 131,072 entries each"}[self.name]
        bt = blas_threads()
        n_cpu, model = cpu_info()
        return {"value": round(rows / dt, 4), "unit": "query-tokens/s", "cores": bt,
                "kind": "oracle", "os_cpu_count": n_cpu, "cpu_model": model,
                "value_1thread": round(1 / dt1, 4),
                "sample": f"{rows} of the {B} sequences of one step ({what}), fp64 numpy with BLAS "
                          f"calls on {bt} threads (element-wise decoding on one): {dt:.1f} s; one "
                          f"sequence with BLAS limited to 1 thread: {dt1:.1f} s"}


# ------------------------------------------------------------------------------------ prefill
class Prefill:
    """c5: T = 4,096 queries at the tail of a 262,144-token context (131,072 entries at 1:2).
    c5r4 (ratio=4): the same 131,072 entries at the predecessor's 4:1 compression, i.e. the
    tail of a 524,288-token context."""

    def __init__(self, args, torch, synth, csa2, dev, ratio=None):
        self.name, self.torch, self.csa2, self.dev = "c5" if ratio is None else "c5r4", torch, csa2, dev
        self.cfg = cfg = dict(synth.CONFIGS["c5_prefill"])
        if ratio is not None:
            cfg["ctx"] = cfg["ctx"] // cfg["ratio"] * ratio
            cfg["ratio"] = ratio
        self.T, self.ratio, self.K = cfg["T"], cfg["ratio"], cfg["k"]
        self.N = cfg["ctx"] // self.ratio
        self.pos0 = cfg["ctx"] - self.T
        n_sets = args.sets or 2
        print(f"generating {n_sets} prefill sets ({self.T} queries, {self.N} entries)",
              file=sys.stderr, flush=True)
        self.sets = []
        for s in range(n_sets):
            seed = cfg["seed"] + 1000 * s
            self.sets.append((synth.make_entries([self.N], seed=seed, device=dev),
                              synth.make_index_queries(self.T, seed, device=dev),
                              synth.make_queries(self.T, seed, device=dev),
                              synth.make_swa(1, self.T + SWA - 1, seed, device=dev)[0]))
        self.idx = torch.empty((self.T, self.K), dtype=torch.int32, device=dev)
        self.out = torch.empty((self.T, HEADS, D_KV), dtype=torch.float32, device=dev)
        self.ws = csa2.prefill_workspace(self.T, self.N, self.K, device=dev)
        self.attn_ws = csa2.attn_workspace(self.T, self.K, device=dev)
        self.stream = torch.cuda.current_stream()
        self.queries_per_step = self.T
        self.n_marks = 3
        self.phase_names = ["indexer_select_us", "attention_us"]
        # visible entry-pairs of the causal contraction: query t sees (pos0 + t + 1) // ratio
        self.pairs = sum(min(self.N, (self.pos0 + t + 1) // self.ratio) for t in range(self.T))

    def step(self, i, marks=None):
        """The chunk as its two halves (the same kernels csa2_prefill_chunk runs): the causal
        indexer and per-query selection, then the attention over the lists."""
        c, qi, q, sw = self.sets[i % len(self.sets)]
        s = self.stream
        m = marks if marks is not None else Marks([None] * 3)
        m[0].record(s)
        self.csa2.csa2_prefill_select(qi, c.idx_codes, c.idx_scale, self.N, self.ratio, self.pos0,
                                      self.K, self.idx, self.ws, stream=s)
        m[1].record(s)
        self.csa2.csa2_sparse_attn_prefill(q, c.kv_codes, c.kv_scale, self.idx, sw, self.pos0,
                                           self.out, self.attn_ws, stream=s)
        m[2].record(s)

    def dominant(self):
        # the causal indexer contraction counted once (2 flops per multiply-add; the library
        # runs a quarter of it again for the sampled threshold), timed over the whole indexer
        # and selection call: a lower bound on the contraction's own rate (per kernel:
        # rocprofv3)
        return {"kernel": "csa2_prefill_select (causal BF16 MFMA indexer contraction, sampled "
                          "threshold and per-query top-512; the call timed)",
                "bound": "mfma", "unit": "TFLOP/s", "peak": BF16_PEAK_TFLOPS,
                "work": 2 * D_IDX * self.pairs, "scale": 1e12, "marks": (0, 1)}

    def step_bytes(self):
        return (self.N * IDX_ENTRY_BYTES + self.T * (D_IDX * 2 + HEADS * D_KV * 2 + HEADS * D_KV * 4 +
                                                     self.K * (MAIN_ENTRY_BYTES + 4) + SWA * D_KV))

    def valid(self):
        return bool(((self.idx[:, 1:] > self.idx[:, :-1]).all() & (self.idx >= 0).all()).item()) and \
            bool(self.torch.isfinite(self.out).all().item())

    def config(self, n_sets):
        ctx = self.cfg["ctx"]
        return {"workload": f"{self.name}_prefill: 4,096 queries at positions {self.pos0:,}..{ctx - 1:,} "
                            f"of a {ctx:,}-token context ({self.N:,} entries at 1:{self.ratio}), causal "
                            "indexer, top-512 per query, attention 16x512 + causal SWA 128",
                "queries": self.T, "context_tokens": self.cfg["ctx"], "entries": self.N,
                "top_k": self.K, "heads": HEADS, "head_dim": D_KV, "swa": SWA,
                "input_sets_rotated": n_sets}

    def cpu_baseline(self, rows):
        import oracle
        c, qi, q, sw = self.sets[0]
        rows = max(1, rows or 4)
        sample = [self.T - 1 - r * (self.T // rows) for r in range(rows)]
        args = (host(qi), host(q), host(c.idx_codes), host(c.idx_scale), host(c.kv_codes),
                host(c.kv_scale), self.N, self.ratio, self.pos0, self.K, host(sw))
        dt = timed_oracle(lambda: oracle.prefill_chunk(*args, rows=sample), None)
        dt1 = timed_oracle(lambda: oracle.prefill_chunk(*args, rows=sample[:1]), 1)
        bt = blas_threads()
        n_cpu, model = cpu_info()
        return {"value": round(rows / dt, 4), "unit": "query-tokens/s", "cores": bt, "kind": "oracle",
                "os_cpu_count": n_cpu, "cpu_model": model, "value_1thread": round(1 / dt1, 4),
                "sample": f"{rows} of the {self.T} queries (spread over the chunk), fp64 numpy with "
                          f"BLAS calls on {bt} threads (element-wise decoding on one): {dt:.1f} s; one "
                          f"query with BLAS limited to 1 thread: {dt1:.1f} s"}


class Model:
    """A whole 40-layer decode step at a 2^20-token context, batch 4: three encoder Full
    layers each scanning its own 524,288-entry pool (1:2), the decoder's Full layer scanning
    1,048,576 entries (ratio 1) into the 16,384 pool and its own top-512, four Reindex
    layers, and 40 attentions (two window-only, 38 over their lists), each with its own
    query and window (compressed_sparse_kv_csa2_amd.model).  With --graph the step is
    captured once into a HIP graph and replayed."""

    B, N_ENC, N_DEC, POOL, K = 4, 1 << 19, 1 << 20, 16384, 512

    def __init__(self, args, torch, synth, csa2, dev):
        from compressed_sparse_kv_csa2_amd import model
        self.torch, self.model = torch, model
        seed = 3
        B = self.B
        print(f"generating the 2^20 model inputs (3 x {B} x {self.N_ENC} + {B} x {self.N_DEC} "
              "entries)", file=sys.stderr, flush=True)
        self.enc = [synth.make_entries([self.N_ENC] * B, seed=seed, device=dev, field_base=10 * (i + 1))
                    for i in range(3)]
        self.dec = synth.make_entries([self.N_DEC] * B, seed=seed, device=dev)
        self.q_idx = {l: synth.make_index_queries(B, seed, device=dev, sub=l) for l in model.SELECTING}
        self.q = torch.stack([synth.make_queries(B, seed, device=dev, sub=l) for l in range(40)]).contiguous()
        self.swa = torch.stack([synth.make_swa(B, SWA, seed, device=dev, sub=l) for l in range(40)]).contiguous()
        self.swa_len = torch.full((B,), SWA, dtype=torch.int32, device=dev)
        self.run = model.DecodePass(B, self.N_ENC, self.N_DEC, self.POOL, self.K, device=dev)
        self.sets = [None]
        self.stream = torch.cuda.current_stream()
        self.queries_per_step = B
        self.n_marks = 4
        self.phase_names = ["encoder_layers_us", "decoder_full_select_us", "decoder_rest_us"]
        self.graph = None
        if args.graph:
            self.run.step(self.enc, self.dec, self.q_idx, self.q, self.swa, self.swa_len, stream=self.stream)
            torch.cuda.synchronize()
            self.graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(self.graph):
                self.run.step(self.enc, self.dec, self.q_idx, self.q, self.swa, self.swa_len,
                              stream=torch.cuda.current_stream())
            torch.cuda.synchronize()

    def step(self, i, marks=None):
        self.run.step(self.enc, self.dec, self.q_idx, self.q, self.swa, self.swa_len,
                      stream=self.stream, marks=marks)

    def graph_timing(self, steps):
        """ms per step of `steps` back-to-back replays of the captured step, and whether the
        last replay's lists and outputs equal an eager step's."""
        t = self.torch
        self.step(0)
        t.cuda.synchronize()
        ref = [self.run.out.clone()] + [v.clone() for v in self.run.lists.values()]
        t.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.graph.replay()
        t.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        got = [self.run.out] + list(self.run.lists.values())
        same = all(bool(t.equal(a, b)) for a, b in zip(ref, got))
        return ms, same

    def dominant(self):
        return {"kernel": "csa2_select_chain: k_fseg<false> + k_fpick<false> (decoder Full scan of "
                          "1,048,576 entries, pool 16,384 and its own top-512); the call timed",
                "bound": "hbm", "unit": "GB/s", "peak": HBM_PEAK_GBS,
                "work": self.B * self.N_DEC * IDX_ENTRY_BYTES, "scale": 1e9, "marks": (1, 2)}

    def step_bytes(self):
        per_q = (3 * self.N_ENC + self.N_DEC) * IDX_ENTRY_BYTES + 8 * D_IDX * 2
        per_q += self.POOL * 4 + 4 * self.POOL * (IDX_ENTRY_BYTES + 4)
        per_q += 38 * self.K * (MAIN_ENTRY_BYTES + 4) + 40 * (SWA * D_KV + HEADS * D_KV * 2 + HEADS * D_KV * 4)
        return self.B * per_q

    def valid(self):
        t = self.torch
        ok = bool(t.isfinite(self.run.out).all().item())
        for lst in self.run.lists.values():
            ok = ok and bool(((lst[:, 1:] > lst[:, :-1]).all() & (lst >= 0).all()).item())
        return ok

    def config(self, n_sets):
        return {"workload": "model_decode: one decode step of all 40 layers at a 2^20-token context, "
                            "batch 4 (3 encoder Full scans of 524,288 entries, decoder Full scan of "
                            "1,048,576 -> pool 16,384, 4 Reindex, 40 attentions 16x512 + SWA 128)",
                "batch": self.B, "context_tokens": 1 << 20, "encoder_entries": self.N_ENC,
                "decoder_entries": self.N_DEC, "pool": self.POOL, "top_k": self.K, "layers": 40,
                "hip_graph": self.graph is not None}

    def cpu_baseline(self, rows):
        import numpy as np
        import oracle
        model = self.model
        t0 = time.perf_counter()
        b = 0
        lists = {}
        for i, l in enumerate(model.ENCODER_FULL):
            c = self.enc[i]
            sl = slice(b * self.N_ENC, (b + 1) * self.N_ENC)
            lists[l] = oracle.topk(oracle.index_scores(host(self.q_idx[l])[b], host(c.idx_codes[sl]),
                                                       host(c.idx_scale[sl])), self.K)
        sl = slice(b * self.N_DEC, (b + 1) * self.N_DEC)
        codes, scale = host(self.dec.idx_codes[sl]), host(self.dec.idx_scale[sl])
        s = oracle.index_scores(host(self.q_idx[20])[b], codes, scale)
        pool = oracle.topk(s, self.POOL)
        lists[20] = pool[oracle.topk(s[pool], self.K)]
        for l in model.REINDEX:
            lists[l], _ = oracle.reindex_layer(host(self.q_idx[l])[b], codes, scale, pool)
        hosts = [(host(c.kv_codes), host(c.kv_scale)) for c in self.enc + [self.dec]]
        q, sw = host(self.q), host(self.swa)
        for l in range(40):
            src = None if l in model.WINDOW_ONLY else model.list_source(l)
            if src is None or src >= model.DECODER_FULL:
                kc, ks = hosts[3]
                base = b * self.N_DEC
            else:
                kc, ks = hosts[model.ENCODER_FULL.index(src)]
                base = b * self.N_ENC
            idx = np.zeros(0, np.int32) if src is None else lists[src]
            oracle.decode_attention(q[l, b], kc, ks, base, idx, sw[l, b], SWA)
        dt = time.perf_counter() - t0
        bt = blas_threads()
        return {"value": round(1 / dt, 4), "unit": "query-tokens/s", "cores": bt, "kind": "oracle",
                "sample": f"1 of the {self.B} sequences through all 40 layers (3 encoder scans of "
                          f"{self.N_ENC} and the decoder scan of {self.N_DEC} entries, pool, 4 "
                          f"Reindex, 40 attentions), fp64 numpy; BLAS calls on {bt} threads, "
                          f"element-wise decoding on one; {dt:.1f} s"}


class Replay:
    """The decoder's bounded replay at a 2^20-token context: the last 128 tokens of one
    sequence through the decoder's 20 layers (compressed_sparse_kv_csa2_amd.model.
    ReplayChunk): per query a Full scan of its visible entries (up to 1,048,576, ratio 1)
    into its own pool of 16,384 and top-512, four Reindex top-512s in its pool, 20
    attentions with causal windows."""

    T, N, POOL, K = 128, 1 << 20, 16384, 512

    def __init__(self, args, torch, synth, csa2, dev):
        from compressed_sparse_kv_csa2_amd import model
        self.torch, self.model = torch, model
        seed = 12
        self.pos0 = self.N - self.T
        print(f"generating the replay inputs ({self.N} entries, {self.T} queries)", file=sys.stderr,
              flush=True)
        self.cache = synth.make_entries([self.N], seed=seed, device=dev)
        self.q_idx = {l: synth.make_index_queries(self.T, seed, device=dev, sub=l)
                      for l in (20,) + model.REINDEX}
        self.q = torch.stack([synth.make_queries(self.T, seed, device=dev, sub=l)
                              for l in range(20, 40)]).contiguous()
        self.swa = torch.stack([synth.make_swa(1, self.T + SWA - 1, seed, device=dev, sub=l)[0]
                                for l in range(20, 40)]).contiguous()
        self.run = model.ReplayChunk(self.T, self.N, self.pos0, self.POOL, self.K, device=dev)
        self.sets = [None]
        self.stream = torch.cuda.current_stream()
        self.queries_per_step = self.T
        self.n_marks = 3
        self.phase_names = ["full_select_us", "reindex_and_attention_us"]

    def step(self, i, marks=None):
        self.run.step(self.cache, self.q_idx, self.q, self.swa, stream=self.stream, marks=marks)

    def dominant(self):
        # the Full selection's call: the causal MFMA contraction writes the 128 x 2^20 score
        # matrix, then the filtered selection reads it; its algorithmic bytes are the keys,
        # read once for all 128 queries (the matrix's write and read are this design's cost)
        return {"kernel": "csa2_replay_select: k_causal_scores (BF16 MFMA score matrix) + "
                          "k_fseg_mat + k_fpick<false> (per-query pool 16,384 and own top-512); "
                          "the call timed",
                "bound": "hbm", "unit": "GB/s", "peak": HBM_PEAK_GBS,
                "work": self.N * IDX_ENTRY_BYTES, "scale": 1e9, "marks": (0, 1)}

    def step_bytes(self):
        scan = self.N * IDX_ENTRY_BYTES  # the keys, read once for all queries
        per_q = self.POOL * 4 + 4 * self.POOL * (IDX_ENTRY_BYTES + 4) + 5 * D_IDX * 2
        per_q += 20 * (self.K * (MAIN_ENTRY_BYTES + 4) + SWA * D_KV + HEADS * D_KV * 6)
        return scan + self.T * per_q

    def valid(self):
        t = self.torch
        ok = bool(t.isfinite(self.run.out).all().item())
        for lst in self.run.lists.values():
            ok = ok and bool(((lst[:, 1:] > lst[:, :-1]).all() & (lst >= 0).all()).item())
        return ok

    def config(self, n_sets):
        return {"workload": "replay: the last 128 tokens of a 2^20-token sequence through the 20 "
                            "decoder layers (per-query Full selection over up to 1,048,576 entries "
                            "-> pool 16,384 + own top-512, 4 Reindex, 20 attentions 16x512 + causal "
                            "SWA 128)",
                "queries": self.T, "context_tokens": self.N, "entries": self.N, "pool": self.POOL,
                "top_k": self.K, "layers": 20}

    def cpu_baseline(self, rows):
        import numpy as np
        import oracle
        t = self.T - 1
        t0 = time.perf_counter()
        codes, scale = host(self.cache.idx_codes), host(self.cache.idx_scale)
        s = oracle.index_scores(host(self.q_idx[20])[t], codes, scale)
        pool = oracle.topk(s, self.POOL)
        lists = {20: pool[oracle.topk(s[pool], self.K)]}
        for l in self.model.REINDEX:
            lists[l], _ = oracle.reindex_layer(host(self.q_idx[l])[t], codes, scale, pool)
        kc, ks, q, sw = host(self.cache.kv_codes), host(self.cache.kv_scale), host(self.q), host(self.swa)
        for l in range(20, 40):
            win = sw[l - 20][t: t + SWA]
            oracle.decode_attention(q[l - 20][t], kc, ks, 0, lists[self.model.list_source(l)], win, SWA)
        dt = time.perf_counter() - t0
        bt = blas_threads()
        return {"value": round(1 / dt, 4), "unit": "query-tokens/s", "cores": bt, "kind": "oracle",
                "sample": f"the last of the {self.T} queries through the 20 decoder layers (scan of "
                          f"{self.N} entries, pool, 4 Reindex, 20 attentions), fp64 numpy; BLAS calls "
                          f"on {bt} threads, element-wise decoding on one; {dt:.1f} s"}


class Append:
    """The KV write path: one layer's new entries for a 262,144-token prompt at 1:2
    (131,072 entries quantised into the 68 B + 288 B formats, written contiguously), and, as
    a separate phase, one new window row for each of 32 sequences."""

    N = 131072
    B_SWA = 32

    def __init__(self, args, torch, synth, csa2, dev):
        self.torch, self.csa2 = torch, csa2
        n_sets = args.sets or 2
        print(f"generating {n_sets} append sets ({self.N} entries)", file=sys.stderr, flush=True)
        self.sets = [synth.make_append_vectors(self.N, seed=50 + s, device=dev) for s in range(n_sets)]
        self.rows = synth.make_window_rows(self.B_SWA, seed=50, device=dev)
        self.pos = torch.arange(1000, 1000 + self.B_SWA, dtype=torch.int64, device=dev)
        self.swa = torch.zeros((self.B_SWA, SWA, D_KV), dtype=torch.uint8, device=dev)
        self.dst = torch.arange(self.N, dtype=torch.int64, device=dev)
        self.planes = (torch.zeros((self.N, 64), dtype=torch.uint8, device=dev),
                       torch.zeros((self.N,), dtype=torch.float32, device=dev),
                       torch.zeros((self.N, 256), dtype=torch.uint8, device=dev),
                       torch.zeros((self.N, 32), dtype=torch.uint8, device=dev))
        self.stream = torch.cuda.current_stream()
        self.queries_per_step = self.N
        self.n_marks = 3
        self.phase_names = ["kv_append_us", "swa_append_us"]

    def step(self, i, marks=None):
        xi, xk = self.sets[i % len(self.sets)]
        s = self.stream
        m = marks if marks is not None else Marks([None] * 3)
        m[0].record(s)
        self.csa2.csa2_kv_append(xi, xk, self.dst, *self.planes, stream=s)
        m[1].record(s)
        self.csa2.csa2_swa_append(self.rows, self.pos, self.swa, stream=s)
        m[2].record(s)

    def entry_bytes(self):
        # read: 128 + 512 bf16 values and the 8-byte id; write: the 68 + 288-byte entry
        return D_IDX * 2 + D_KV * 2 + 8 + IDX_ENTRY_BYTES + MAIN_ENTRY_BYTES

    def dominant(self):
        return {"kernel": "k_kv_append (quantise 131,072 entries into the 68 B + 288 B formats)",
                "bound": "hbm", "unit": "GB/s", "peak": HBM_PEAK_GBS,
                "work": self.N * self.entry_bytes(), "scale": 1e9, "marks": (0, 1)}

    def step_bytes(self):
        return self.N * self.entry_bytes() + self.B_SWA * (D_KV * 2 + 8 + D_KV)

    def valid(self):
        return bool((self.planes[1] > 0).all().item())

    def config(self, n_sets):
        return {"workload": "kv_append: 131,072 new entries (one layer of a 262,144-token prompt "
                            "at 1:2) quantised and written contiguously, plus one window row for "
                            "each of 32 sequences",
                "entries": self.N, "window_rows": self.B_SWA, "input_sets_rotated": n_sets}

    def cpu_baseline(self, rows):
        import numpy as np
        import oracle
        xi, xk = self.sets[0]
        rows = rows or 16384
        hi, hk = host(xi[:rows]), host(xk[:rows])
        z = (np.zeros((rows, 64), np.uint8), np.zeros(rows, np.float32),
             np.zeros((rows, 256), np.uint8), np.zeros((rows, 32), np.uint8))
        t0 = time.perf_counter()
        oracle.kv_append(*z, hi, hk, np.arange(rows))
        dt = time.perf_counter() - t0
        return {"value": round(rows / dt, 1), "unit": "entries/s", "cores": 1, "kind": "oracle",
                "sample": f"the first {rows} of the {self.N} entries, fp64/fp32 numpy on one "
                          f"thread; {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "split of this path is a design, not a build", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.read_probe:
        read_probe(args.read_probe)
        return

    import torch
    import synth
    import compressed_sparse_kv_csa2_amd as csa2

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X", file=sys.stderr)
        sys.exit(1)
    csa2.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.workload in ("c5", "c5r4"):
        wl = Prefill(args, torch, synth, csa2, dev, ratio=4 if args.workload == "c5r4" else None)
    elif args.workload == "append":
        wl = Append(args, torch, synth, csa2, dev)
    elif args.workload == "model":
        wl = Model(args, torch, synth, csa2, dev)
    elif args.workload == "replay":
        wl = Replay(args, torch, synth, csa2, dev)
    else:
        wl = Decode(args.workload, args, torch, synth, csa2, dev)
    torch.cuda.synchronize()
    print("inputs ready", file=sys.stderr, flush=True)

    for i in range(args.warmup):
        wl.step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps; the dominant launch bracketed by events
    dom = wl.dominant()
    a, b = dom["marks"]
    marks = [Marks([torch.cuda.Event(enable_timing=True) if j in (a, b) else None
                    for j in range(wl.n_marks)]) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        wl.step(i, marks[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    dom_ms = sum(m[a].elapsed_time(m[b]) for m in marks) / args.steps
    achieved = dom["work"] / (dom_ms * 1e-3) / dom["scale"]
    ms_per_step = elapsed * 1e3 / args.steps
    value = wl.queries_per_step * args.steps / elapsed
    step_bytes = wl.step_bytes()
    step_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9

    phases = None
    if not args.no_phases:
        reps = max(20, min(100, args.steps))
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(wl.n_marks)] for _ in range(reps)]
        for i in range(reps):
            wl.step(i, Marks(evs[i]))
        torch.cuda.synchronize()
        phases = {n: round(sum(e[j].elapsed_time(e[j + 1]) for e in evs) * 1e3 / reps, 2)
                  for j, n in enumerate(wl.phase_names) if n}

    torch.cuda.synchronize()
    ok = wl.valid()
    print(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step", file=sys.stderr, flush=True)
    cpu = None if args.no_cpu_baseline else wl.cpu_baseline(args.cpu_rows)

    headline = args.workload == "c4"
    line = {
        "metric": METRIC if headline else
        {"c2": "CSA2 batched Full decode query-tokens/s (32 x 32,768 entries)",
         "c3": "CSA2 decoder-chain query-tokens/s (20 layers, 16 x 131,072 entries)",
         "c5": "CSA2 prefill query-tokens/s (4,096-query chunk, 131,072 entries)",
         "c5r4": "CSA2 prefill query-tokens/s at 4:1 compression (4,096-query chunk, 131,072 entries)",
         "append": "CSA2 KV append entries/s (131,072 entries)",
         "model": "CSA2 whole-model decode query-tokens/s (40 layers, 2^20 ctx, batch 4)",
         "replay": "CSA2 decoder replay query-tokens/s (128 tokens, 20 layers, 2^20 ctx)"}[args.workload],
        "value": round(value, 1),
        "unit": "entries/s" if args.workload == "append" else "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": wl.config(len(wl.sets)),
        "roofline": {"kernel": dom["kernel"], "bound": dom["bound"], "achieved": round(achieved, 1),
                     "peak": dom["peak"], "unit": dom["unit"],
                     "frac": round(achieved / dom["peak"], 4),
                     "traffic": read_traffic() if headline and args.select == "chain" else None,
                     "algorithmic_per_launch": dom["work"],
                     "avg_launch_us": round(dom_ms * 1e3, 2)},
        "step_hbm": {"algorithmic_bytes": step_bytes, "achieved_gbs": round(step_gbs, 1),
                     "frac": round(step_gbs / HBM_PEAK_GBS, 4)},
        "phases_us": phases,
        "selection_valid": ok,
        "cpu_baseline": cpu,
    }
    if getattr(wl, "status", None) is not None:
        line["workspace_status"] = [{"error_bits": b, "rows_rescanned": n} for b, n in wl.status]
    if headline and args.select == "chain" and not args.no_per_layer:
        pl = wl.per_layer(args.steps)
        line["per_layer_path"] = pl
        ok = ok and pl["valid"]
    if getattr(wl, "graph", None) is not None:
        g_ms, g_same = wl.graph_timing(args.steps)
        line["hip_graph"] = {"ms_per_step": round(g_ms, 5),
                             "value": round(wl.queries_per_step / (g_ms * 1e-3), 1),
                             "replays_equal_eager": g_same}
        ok = ok and g_same
    print(json.dumps(line), flush=True)
    if not ok:
        sys.exit(3)


if __name__ == "__main__":
    main()
