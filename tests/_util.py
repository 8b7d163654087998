"""Shared test helpers: fixture reader and the parity rules used by GPU tests."""
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def read_golden(name):
    """Parse a whitespace fixture: '#' comments, then 'key value...' lines."""
    rows = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------------------- parity rules
TOPK_GAP = 1e-4      # relative k-th / (k+1)-th gap above which sets must match exactly
ATTN_TOL = 2e-3      # max over (query, head) of ||gpu - ref||_inf / ||ref||_inf


def check_topk(gpu_idx, ref_scores, k, ids=None, n_valid=None, label=""):
    """Top-k parity rule against fp64 oracle scores.

    gpu_idx: the GPU's list (ascending ids, -1 padded).  ref_scores[c]: oracle score of
    column c; ids[c]: entry id of column c (default c).  Where the oracle's k-th/(k+1)-th
    relative gap exceeds TOPK_GAP the sets must be equal; otherwise every id in the
    symmetric difference must score within TOPK_GAP*|s_k| of s_k.  Returns the gap."""
    s = np.asarray(ref_scores, dtype=np.float64)
    n = s.shape[0] if n_valid is None else int(n_valid)
    s = s[:n]
    ids = np.arange(n) if ids is None else np.asarray(ids)[:n]
    g = np.asarray(gpu_idx)
    m = min(k, n)
    assert np.all(g[m:] == -1), f"{label}: padding wrong"
    got = g[:m]
    assert np.all(got >= 0), f"{label}: missing entries"
    assert np.all(np.diff(got) > 0), f"{label}: not strictly ascending"
    assert set(got.tolist()) <= set(ids.tolist()), f"{label}: ids outside the candidate set"
    order = np.lexsort((ids, -s))
    want = np.sort(ids[order[:m]])
    if m == n:
        assert np.array_equal(got, want), f"{label}: all columns should be selected"
        return np.inf
    sk, sk1 = s[order[m - 1]], s[order[m]]
    gap = (sk - sk1) / abs(sk) if sk != 0 else (np.inf if sk1 < sk else 0.0)
    if gap > TOPK_GAP:
        assert np.array_equal(got, want), f"{label}: sets differ with gap {gap:.3g}"
    else:
        score_of = dict(zip(ids.tolist(), s.tolist()))
        diff = set(got.tolist()) ^ set(want.tolist())
        tol = TOPK_GAP * abs(sk)
        bad = [j for j in diff if abs(score_of[j] - sk) > tol]
        assert not bad, f"{label}: {len(bad)} ids outside the tie band (gap {gap:.3g})"
    return gap


def attn_rel_err(gpu, ref):
    """max over (query, head) of ||gpu - ref||_inf / ||ref||_inf."""
    gpu = np.asarray(gpu, dtype=np.float64).reshape(-1, 512)
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, 512)
    num = np.abs(gpu - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


def score_error_bound(q_bits, codes, scale):
    """|fp32-accumulated score - exact| bound for 128-term dots of exact products:
    127 * 2^-24 * scale * sum|q_d v_d| plus one rounding of the scaled result."""
    from oracle import formats
    q = formats.bf16_decode(q_bits)
    v = formats.e2m1_decode(formats.unpack_nibbles(codes))
    mag = np.abs(v) @ np.abs(q)
    sc = np.asarray(scale, np.float32).astype(np.float64)
    exact = sc * (v @ q)
    return 130 * 2.0 ** -24 * sc * mag + 2.0 ** -23 * np.abs(exact)


def assert_ws_ok(*workspaces):
    """Every selection workspace's status block reports no error bits."""
    import compressed_sparse_kv_csa2_amd as csa2
    for ws in workspaces:
        bits, _ = csa2.csa2_workspace_status(ws)
        assert bits == 0, f"selection workspace error bits {bits:#x}"
