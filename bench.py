"""Throughput of the CSA2 decode step on one MI355X, with its HBM roofline and the CPU oracle.

One step is the decoder step at a 2^20-token context for a batch of 4 sequences:
  Full scan of 1,048,576 FP4 indexer keys per sequence (csa2_index_score, fused level-1
  radix histogram) -> candidate pool of 16,384 (csa2_topk) -> Reindex re-score of the pool
  with the next layer's indexer query (csa2_index_score over the pool) -> its top-512
  (csa2_topk) -> gather-dequant attention of 16 heads x 512 merged with a 128-row FP8
  window (csa2_sparse_attn_decode).
Layer modes and pool: "DeepSeek-V4.1 模型结构（0）：一张图看懂 DeepSeek-V4.1-Flash", commentary
on the four layer modes; "从V4到V4.1 Flash：架构的激进进化", decoder section (a first full scan
builds a pool of about 16K positions; later layers pick their top-512 inside it).

Inputs are seeded synthetic N(0,1) values quantised to the entry formats (synth.py), already
resident in HBM when timing starts.  Several independent input sets are rotated step by
step so that the caches never hold the bytes a step reads (a set's indexer keys alone are
285 MB, more than the 256 MiB last-level cache).

Prints ONE JSON line.  `roofline` is for the dominant kernel (the Full scan): algorithmic
bytes (68 B per scanned entry) per launch divided by its average launch time, measured
with events on the launch stream inside the timed region.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "CSA2 decode query-tokens/s at 2^20 ctx; achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
IDX_ENTRY_BYTES = 68         # 128 x 4 bit + 4-byte scale
MAIN_ENTRY_BYTES = 288       # 512 x 4 bit + 32 E4M3 scale bytes
D_KV, HEADS, SWA = 512, 16, 128
SCAN_SOURCES = ("compressed_sparse_kv_csa2_amd/csrc/index_score.hip",
                "compressed_sparse_kv_csa2_amd/csrc/csa2_device.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_index_score_c4_long_decode_traffic.md")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--sets", type=int, default=4, help="independent input sets rotated per step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=2,
                   help="sequences of the first input set the CPU oracle runs")
    p.add_argument("--no-phases", action="store_true",
                   help="skip the separate, untimed per-phase timing pass")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="instead of the step, run 5 plain device copies of MIB MiB (the known-size "
                        "reference for scaling the HBM counters) and exit")
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


def scan_source_digest() -> str:
    h = hashlib.sha256()
    for rel in SCAN_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per scan launch from the committed rocprofv3 counter summary, or None when
    the summary is absent or was taken on a different version of the scan kernel."""
    try:
        text = open(TRAFFIC_FILE, encoding="utf-8").read()
    except OSError:
        return None
    m_src = re.search(r"source_digest:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_b or m_src.group(1) != scan_source_digest():
        return None
    return float(m_b.group(1))


class Workload:
    """One input set of the 2^20-context decoder step: B sequences x N decoder entries."""

    def __init__(self, synth, torch, B, N, seed, dev):
        self.cache = synth.make_entries([N] * B, seed=seed, device=dev)
        self.q_full = synth.make_index_queries(B, seed, device=dev, sub=20)
        self.q_re = synth.make_index_queries(B, seed, device=dev, sub=24)
        self.q = synth.make_queries(B, seed, device=dev, sub=24)
        self.swa = synth.make_swa(B, SWA, seed, device=dev, sub=24)
        self.swa_len = torch.full((B,), SWA, dtype=torch.int32, device=dev)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "split of this path is a design, not a build", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
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

    cfg = synth.CONFIGS["c4_long_decode"]
    B, N, POOL, K = cfg["B"], cfg["ctx"] // cfg["ratio"], cfg["pool"], cfg["k"]
    print(f"generating {args.sets} input sets of {B} x {N} entries", file=sys.stderr, flush=True)
    sets = [Workload(synth, torch, B, N, cfg["seed"] + 1000 * s, dev) for s in range(args.sets)]
    torch.cuda.synchronize()
    print("inputs ready", file=sys.stderr, flush=True)

    # Preallocated outputs and workspaces (the library allocates nothing).
    ws = [csa2.topk_workspace(B, N, POOL, device=dev) for _ in sets]
    scores = torch.empty((B, N), dtype=torch.float32, device=dev)
    pool = torch.empty((B, POOL), dtype=torch.int32, device=dev)
    rescore = torch.empty((B, POOL), dtype=torch.float32, device=dev)
    idx = torch.empty((B, K), dtype=torch.int32, device=dev)
    out = torch.empty((B, HEADS, D_KV), dtype=torch.float32, device=dev)
    attn_ws = csa2.attn_workspace(B, K, device=dev)
    pool_valid = torch.full((B,), POOL, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        w, tw = sets[i % len(sets)], ws[i % len(sets)]
        c = w.cache
        if ev is not None:
            ev[0].record(stream)
        csa2.csa2_index_score(w.q_full, c.idx_codes, c.idx_scale, c.seq_base, c.n_entries, scores,
                              topk_ws=tw, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        csa2.csa2_topk(scores, c.n_entries, POOL, pool, hist_fused=True, workspace=tw, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        csa2.csa2_index_score(w.q_re, c.idx_codes, c.idx_scale, c.seq_base, pool_valid, rescore,
                              cand=pool, stream=stream)
        csa2.csa2_topk(rescore, pool_valid, K, idx, cand=pool, stream=stream)
        if ev is not None:
            ev[3].record(stream)
        csa2.csa2_sparse_attn_decode(w.q, c.kv_codes, c.kv_scale, c.seq_base, idx, w.swa, w.swa_len,
                                     out, attn_ws, stream=stream)
        if ev is not None:
            ev[4].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps; scan launches bracketed by events
    scan_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        w, tw = sets[i % len(sets)], ws[i % len(sets)]
        c = w.cache
        scan_ev[i][0].record(stream)
        csa2.csa2_index_score(w.q_full, c.idx_codes, c.idx_scale, c.seq_base, c.n_entries, scores,
                              topk_ws=tw, stream=stream)
        scan_ev[i][1].record(stream)
        csa2.csa2_topk(scores, c.n_entries, POOL, pool, hist_fused=True, workspace=tw, stream=stream)
        csa2.csa2_index_score(w.q_re, c.idx_codes, c.idx_scale, c.seq_base, pool_valid, rescore,
                              cand=pool, stream=stream)
        csa2.csa2_topk(rescore, pool_valid, K, idx, cand=pool, stream=stream)
        csa2.csa2_sparse_attn_decode(w.q, c.kv_codes, c.kv_scale, c.seq_base, idx, w.swa, w.swa_len,
                                     out, attn_ws, stream=stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    ms_per_step = elapsed * 1e3 / args.steps
    value = B * args.steps / elapsed
    scan_ms = sum(a.elapsed_time(b) for a, b in scan_ev) / args.steps
    scan_bytes = B * N * IDX_ENTRY_BYTES
    achieved = scan_bytes / (scan_ms * 1e-3) / 1e9
    traffic = read_traffic()

    # Bytes the whole step must move (per query: scan, pool re-score with its index list,
    # 512 gathered main entries with their index, the window, q and the output).
    step_bytes = B * (N * IDX_ENTRY_BYTES + POOL * (IDX_ENTRY_BYTES + 4) +
                      K * (MAIN_ENTRY_BYTES + 4) + SWA * D_KV + HEADS * D_KV * 2 + 256 * 2 +
                      HEADS * D_KV * 4 + POOL * 4)
    step_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9

    phases = None
    if not args.no_phases:
        reps = max(20, min(100, args.steps))
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(reps)]
        for i in range(reps):
            step(i, evs[i])
        torch.cuda.synchronize()
        names = ["scan_us", "pool_topk_us", "reindex_us", "attention_us"]
        phases = {n: round(sum(e[j].elapsed_time(e[j + 1]) for e in evs) * 1e3 / reps, 2)
                  for j, n in enumerate(names)}

    # Correctness guard: the last step's selection must be a valid ascending list.
    torch.cuda.synchronize()
    ok = bool(((idx[:, 1:] > idx[:, :-1]).all() & (idx >= 0).all()).item()) and \
        bool(torch.isfinite(out).all().item())

    print(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(sets[0], B, N, POOL, K, args.cpu_rows)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "c4_long_decode: decoder step at 2^20 ctx, batch 4, Full scan of "
                               "1,048,576 entries -> pool 16,384 -> Reindex top-512 -> "
                               "attention 16x512 + SWA 128",
                   "batch": B, "context_tokens": cfg["ctx"], "decoder_entries": N,
                   "pool": POOL, "top_k": K, "heads": HEADS, "head_dim": D_KV, "swa": SWA,
                   "input_sets_rotated": args.sets},
        "roofline": {"kernel": "k_index_score (Full scan)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": scan_bytes,
                     "avg_launch_us": round(scan_ms * 1e3, 2)},
        "step_hbm": {"algorithmic_bytes": step_bytes, "achieved_gbs": round(step_gbs, 1),
                     "frac": round(step_gbs / HBM_PEAK_GBS, 4)},
        "phases_us": phases,
        "selection_valid": ok,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    if not ok:
        sys.exit(3)


def cpu_baseline(w, B, N, POOL, K, rows):
    """The fp64 oracle on the host: the same decoder step for `rows` sequences of the first
    input set, timed around the oracle calls only."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()
                            if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: numpy's BLAS pool size unknown
        blas_threads = 1

    def h(t):
        a = t.detach().cpu().numpy()
        return a.view(np.uint16) if a.dtype == np.int16 else a

    c = w.cache
    rows = max(1, min(rows, B))
    data = dict(codes=h(c.idx_codes[: rows * N]), scale=h(c.idx_scale[: rows * N]),
                kvc=h(c.kv_codes[: rows * N]), kvs=h(c.kv_scale[: rows * N]),
                qf=h(w.q_full), qr=h(w.q_re), q=h(w.q), swa=h(w.swa))
    t0 = time.perf_counter()
    for b in range(rows):
        oracle.decode_step_long(data["qf"][b], data["qr"][b], data["q"][b], data["codes"],
                                data["scale"], data["kvc"], data["kvs"], b * N, N, data["swa"][b],
                                SWA, POOL, K)
    dt = time.perf_counter() - t0
    return {"value": round(rows / dt, 4), "unit": "query-tokens/s", "cores": blas_threads,
            "kind": "oracle",
            "sample": f"{rows} of the {B} sequences of one step (full 1,048,576-entry scan, pool, "
                      f"Reindex, attention each), fp64 numpy; BLAS calls on {blas_threads} "
                      f"threads, element-wise decoding on one; {dt:.1f} s"}


if __name__ == "__main__":
    main()
