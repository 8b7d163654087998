"""csa2_sparse_attn_decode_noalloc (split partials in the library's static scratch, no
allocation) against csa2_sparse_attn_decode (the caller's workspace), through the C ABI:
the same kernels, so the outputs must agree bit for bit, on two calls in a row, the
second with a smaller input (the scratch keeps the first call's partials)."""
import math
import sys

import numpy as np
import pytest
import torch

import compressed_sparse_kv_csa2_amd as csa2
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCALE = 1.0 / math.sqrt(512)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(B, n, k, seed):
    cache = synth.make_entries([n] * B, seed=seed, device=DEV)
    q = synth.make_queries(B, seed, device=DEV)
    swa = synth.make_swa(B, 128, seed, device=DEV)
    rng = np.random.default_rng(seed)
    idx = np.stack([np.sort(rng.choice(n, k, replace=False)) for _ in range(B)]).astype(np.int32)
    idx[B - 1, ::5] = -1                      # holes in the last row's list
    lens = np.full(B, 128, np.int32)
    lens[0] = 77                              # a short window
    return cache, q, swa, torch.from_numpy(idx).to(DEV), torch.from_numpy(lens).to(DEV)


@pytest.mark.parametrize("first,second", [((8, 6000, 2048), (4, 3000, 512))])
def test_noalloc_matches_workspace_entry_point(first, second):
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    lib = csa2.load_library()
    for i, (B, n, k) in enumerate((first, second)):
        log(f"noalloc call {i}: B={B} n={n} k={k}")
        assert lib.csa2_attn_workspace_size(B, k) > 256, "the shape must use split partials"
        assert lib.csa2_attn_workspace_size(B, k) <= lib.csa2_attn_noalloc_max_bytes()
        cache, q, swa, idx, lens = _inputs(B, n, k, 31 + i)
        out_ws = torch.empty((B, 16, 512), dtype=torch.float32, device=DEV)
        out_na = torch.full((B, 16, 512), float("nan"), dtype=torch.float32, device=DEV)
        ws = csa2.attn_workspace(B, k, device=DEV)
        csa2.csa2_sparse_attn_decode(q, cache.kv_codes, cache.kv_scale, cache.seq_base, idx, swa, lens,
                                     out_ws, ws, softmax_scale=SCALE)
        csa2.csa2_sparse_attn_decode_noalloc(q, cache.kv_codes, cache.kv_scale, cache.seq_base, idx, swa,
                                             lens, out_na, softmax_scale=SCALE)
        torch.cuda.synchronize()
        assert torch.isfinite(out_na).all()
        assert torch.equal(out_na, out_ws), f"call {i}: outputs differ"
