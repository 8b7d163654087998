"""GPU parity of the KV write path (csa2_kv_append, csa2_swa_append) against the CPU
oracle's quantisers, through the C ABI.  Integer/byte output: every plane must match the
oracle bit for bit, at small sizes with crafted edge values and at the benchmark's size
(131,072 entries, the entries one layer holds for a 262,144-token context at 1:2).
"""
import sys

import numpy as np
import pytest
import torch

import compressed_sparse_kv_csa2_amd as csa2
import oracle
import synth

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


def bits(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16)


def planes(cap, fill=0):
    return (torch.full((cap, 64), fill, dtype=torch.uint8, device=DEV),
            torch.full((cap,), float(fill), dtype=torch.float32, device=DEV),
            torch.full((cap, 256), fill, dtype=torch.uint8, device=DEV),
            torch.full((cap, 32), fill, dtype=torch.uint8, device=DEV))


def run_and_check(x_idx, x_kv, dst, cap, fill=0):
    p = planes(cap, fill)
    before = [h(t) for t in p]
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    csa2.csa2_kv_append(x_idx.to(DEV), x_kv.to(DEV), torch.tensor(dst, dtype=torch.int64, device=DEV),
                        *p, bad=bad)
    torch.cuda.synchronize()
    ic, isc, kc, ksc, nbad = oracle.kv_append(*before, h(x_idx), h(x_kv), dst)
    assert int(h(bad)[0]) == nbad
    assert np.array_equal(h(p[0]), ic), "indexer codes"
    assert np.array_equal(h(p[1]).view(np.uint32), isc.view(np.uint32)), "indexer scales"
    assert np.array_equal(h(p[2]), kc), "main codes"
    assert np.array_equal(h(p[3]), ksc), "main scales"


def test_append_random_scatter_with_rejected_ids():
    log("kv_append scatter n=1000")
    n, cap = 1000, 1500
    x_idx, x_kv = synth.make_append_vectors(n, seed=21)
    rng = np.random.default_rng(21)
    dst = rng.permutation(cap)[:n].astype(np.int64)
    dst[[5, 77, 400]] = [-3, cap, cap + 1000]
    run_and_check(x_idx, x_kv, dst, cap, fill=0xAB)


def test_append_edge_values():
    log("kv_append edge values")
    rows_i, rows_k = [], []
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    # scale exactly 1: every E2M1 midpoint tie, both signs, on both planes
    r = np.zeros(128); r[0] = 6.0; r[1:8] = mids; r[8:15] = [-m for m in mids]; r[15] = -0.0
    rows_i.append(r)
    k = np.tile(np.r_[6.0, mids, [-m for m in mids], -0.0], 32)
    rows_k.append(k)
    # all zero (indexer scale 1, main scale code 1) and negative zeros
    rows_i.append(-np.zeros(128)); rows_k.append(-np.zeros(512))
    # saturating main scales (amax/6 > 448), huge indexer values
    rows_i.append(np.full(128, 3e37) * np.resize([1, -1, 0.5, 0.1], 128))
    rows_k.append(np.resize([3e4, -1e4, 7.0, 0.01], 512))
    # quotients far beyond 6 (saturated scales with huge values)
    rows_i.append(np.resize([1.0, -2.0], 128))
    rows_k.append(np.resize([1e37, -3e38, 1.0, 0.0], 512))
    # tiny values: E4M3 subnormal scales, values that vanish, bf16 subnormals in a group
    rows_i.append(np.resize([1e-30, -3e-31, 2e-32, 1e-40], 128))
    rows_k.append(np.resize([1e-5, -2e-6, 3e-7, 1e-40, 5e-4, -7e-5, 2.2e-3, 0.0], 512))
    # scales on E4M3 midpoints: amax/6 exactly between two E4M3 values
    rows_i.append(np.linspace(-1, 1, 128) * 3.1)
    rows_k.append(np.resize([6 * 1.0625, 6 * 1.1875, 6 * (2 ** -7 + 2 ** -10), 1.0], 512))
    x_idx, x_kv = bits(np.array(rows_i)), bits(np.array(rows_k))
    n = x_idx.shape[0]
    run_and_check(x_idx, x_kv, np.arange(n, dtype=np.int64)[::-1].copy(), n)


def test_append_benchmark_size():
    # the benchmark's batch: 131,072 entries, every plane compared in full
    n = 131072
    log(f"kv_append n={n}")
    x_idx, x_kv = synth.make_append_vectors(n, seed=5, device=DEV)
    dst = np.arange(n, dtype=np.int64)
    run_and_check(x_idx.cpu(), x_kv.cpu(), dst, n)


def test_swa_append_ring():
    log("swa_append ring")
    B = 40
    rng = np.random.default_rng(4)
    swa = synth.make_swa(B, 128, seed=9, device=DEV)
    before = h(swa)
    pos = rng.integers(-5, 100000, B).astype(np.int64)
    pos[:4] = [0, 127, 128, -1]
    x = synth.make_window_rows(B, seed=9, device=DEV)
    x[0, :8] = bits([448.0, 460.0, 470.0, 1e5, -1e5, 2.0 ** -10, 3 * 2.0 ** -11, -0.0]).to(DEV)
    csa2.csa2_swa_append(x, torch.tensor(pos, device=DEV), swa)
    torch.cuda.synchronize()
    want = oracle.swa_append(before, h(x), pos)
    assert np.array_equal(h(swa), want)
