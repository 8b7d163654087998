"""The C-ABI library loads, exports every symbol include/csa2.h declares, and rejects bad
arguments on the host before anything is launched (runs without a GPU: no call here
reaches a kernel)."""
import ctypes
import os
import re

import pytest

import compressed_sparse_kv_csa2_amd as csa2
from _util import ROOT

HEADER = os.path.join(ROOT, "include", "csa2.h")


def _declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(csa2.lib_path):
        pytest.fail("libcsa2.so is not built; run `python -m compressed_sparse_kv_csa2_amd.build`")
    return csa2.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert {"csa2_index_score", "csa2_topk", "csa2_sparse_attn_decode",
            "csa2_prefill_chunk"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared but not exported"
    # and the binding wraps the four path calls under the same names
    for n in ("csa2_index_score", "csa2_topk", "csa2_sparse_attn_decode", "csa2_prefill_chunk"):
        assert callable(getattr(csa2, n))


def test_status_strings_and_version(lib):
    assert lib.csa2_status_string(0) == b"ok"
    for s in range(-6, 0):
        assert lib.csa2_status_string(s) not in (b"ok", b"unknown status")
    assert lib.csa2_status_string(-99) == b"unknown status"
    assert lib.csa2_version() >= 100


def test_workspace_sizes(lib):
    a = lib.csa2_topk_workspace_size(4, 1 << 20, 16384)
    b = lib.csa2_topk_workspace_size(4, 1 << 19, 16384)
    assert a > b > 0
    assert lib.csa2_topk_workspace_size(0, 10, 1) == 0
    assert lib.csa2_attn_workspace_size(4, 512) > lib.csa2_attn_workspace_size(4, 0) > 0
    assert lib.csa2_prefill_workspace_size(4096, 131072, 512) > 0
    assert lib.csa2_prefill_workspace_size(0, 131072, 512) == 0


def test_attention_split_counts(lib):
    # the attention workspace holds one partial (max[16], sum[16], acc[16][512] in fp32) per
    # split and row, so its size gives the split count the launch uses: few rows get the
    # fewest segments per split that leave every split its own compute unit, many rows the
    # square-root rule, and no row is ever cut into more than 64 splits
    part = (2 * 16 + 16 * 512) * 4

    def splits(rows, k):
        size = lib.csa2_attn_workspace_size(rows, k)
        if size == 256:
            return 1
        assert size % 256 == 0 and size >= rows * part
        return size // (rows * part)

    assert [splits(r, 512) for r in (1, 4, 8, 16, 32, 128, 4096)] == [40, 40, 20, 14, 8, 8, 1]
    for rows in (1, 3, 4, 7, 13, 16, 33, 64, 128, 1000):
        for k in (0, 16, 100, 512, 2048, 16384):
            n = splits(rows, k)
            segs = (k + 128 + 15) // 16
            assert 1 <= n <= min(64, segs)
            if rows * segs <= 256 and segs <= 64:
                assert n == segs  # one segment per split when every split gets a unit


FAKE = ctypes.c_void_p(1 << 20)        # never dereferenced: validation fails first
ODD = ctypes.c_void_p((1 << 20) + 2)   # misaligned


def test_index_score_validation(lib):
    f = lib.csa2_index_score
    args = [FAKE] * 6 + [4, 1024, FAKE, None, 0, None]
    bad = list(args); bad[0] = None
    assert f(*bad) == -1
    bad = list(args); bad[6] = 0
    assert f(*bad) == -1
    bad = list(args); bad[1] = ODD
    assert f(*bad) == -2
    bad = list(args); bad[9] = FAKE; bad[10] = 16
    assert f(*bad) == -3


def test_topk_validation(lib):
    f = lib.csa2_topk
    base = [FAKE, 4, 1 << 20, FAKE, None, 512, FAKE, None, 0, FAKE, 1 << 40, None]
    for pos, val, want in [(5, 0, -1), (5, 16385, -1), (0, None, -1), (8, 7, -1), (0, ODD, -2),
                           (10, 100, -3)]:
        a = list(base); a[pos] = val
        assert f(*a) == want, (pos, val)
    a = list(base); a[9] = None
    assert f(*a) == -3  # long rows need a workspace


def test_attn_validation(lib):
    f = lib.csa2_sparse_attn_decode
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, 512, FAKE, FAKE, 0.04, 4, FAKE, FAKE, 1 << 40, None]
    for pos, val, want in [(5, -1, -1), (4, None, -1), (9, 0, -1), (0, ODD, -2), (12, 10, -3)]:
        a = list(base); a[pos] = val
        assert f(*a) == want, (pos, val)


def test_attn_noalloc_validation(lib):
    # the same checks as csa2_sparse_attn_decode, and SCRATCH (-6) for a shape whose split
    # partials (64 rows x 16,384 entries: about 34 MB) exceed the static scratch
    f = lib.csa2_sparse_attn_decode_noalloc
    assert lib.csa2_attn_noalloc_max_bytes() == 16 << 20
    assert lib.csa2_attn_workspace_size(64, 16384) > lib.csa2_attn_noalloc_max_bytes()
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, 16384, FAKE, FAKE, 0.04, 64, FAKE, None]
    for pos, val, want in [(5, -1, -1), (4, None, -1), (9, 0, -1), (0, ODD, -2), (9, 64, -6)]:
        a = list(base); a[pos] = val
        assert f(*a) == want, (pos, val)


def test_prefill_validation(lib):
    f = lib.csa2_prefill_chunk
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 131072, 2, 258048, 4096, 512, FAKE, 0.04, FAKE,
            FAKE, FAKE, 1 << 40, None]
    for pos, val, want in [(7, 0, -1), (8, -1, -1), (10, 0, -1), (9, 0, -1), (1, ODD, -2),
                           (16, 10, -3)]:
        a = list(base); a[pos] = val
        assert f(*a) == want, (pos, val)


def test_index_topk_validation(lib):
    f = lib.csa2_index_topk
    base = [FAKE] * 6 + [4, 1 << 20, 16384, FAKE, None, FAKE, 1 << 40, None]
    for pos, val, want in [(8, 0, -1), (8, 16385, -1), (6, 0, -1), (0, None, -1), (9, None, -1),
                           (1, ODD, -2), (11, None, -3), (12, 100, -3), (7, (1 << 26) + 1, -4)]:
        a = list(base); a[pos] = val
        assert f(*a) == want, (pos, val)
    assert lib.csa2_index_topk_workspace_size(0, 10, 1) == 0
    assert lib.csa2_index_topk_workspace_size(4, 1 << 20, 16384) > 0


def test_select_chain_validation(lib):
    f = lib.csa2_select_chain
    base = [FAKE] * 5 + [4, 1 << 20, 16384, FAKE, None, 512, None, FAKE, 1, FAKE, None, FAKE,
                         1 << 40, None]
    for pos, val, want in [(7, 0, -1), (7, 16385, -1), (10, 0, -1), (13, 5, -1), (13, -1, -1),
                           (12, None, -1), (14, None, -1), (8, None, -1), (0, ODD, -2),
                           (17, 100, -3), (16, None, -3), (6, (1 << 26) + 1, -4)]:
        a = list(base); a[pos] = val
        assert f(*a) == want, (pos, val)
    a = list(base); a[12] = None; a[13] = 0; a[14] = None
    assert f(*a[:17] + [100, None]) == -3  # no Reindex layer: still needs its workspace
    assert lib.csa2_select_chain_workspace_size(4, 1 << 20, 0) == 0
    assert lib.csa2_select_chain_workspace_size(4, 1 << 20, 16384) > 0


def test_kv_append_validation(lib):
    f = lib.csa2_kv_append
    base = [FAKE, FAKE, FAKE, 8, FAKE, FAKE, FAKE, FAKE, 1000, None, None]
    for pos, val, want in [(3, -1, -1), (8, 0, -1), (0, None, -1), (6, None, -1), (1, ODD, -2),
                           (4, ODD, -2)]:
        a = list(base); a[pos] = val
        assert f(*a) == want, (pos, val)
    a = list(base); a[3] = 0; a[0] = None
    assert f(*a) == 0  # n = 0 launches nothing


def test_swa_append_validation(lib):
    f = lib.csa2_swa_append
    base = [FAKE, FAKE, 4, FAKE, None]
    for pos, val, want in [(2, -1, -1), (0, None, -1), (3, None, -1), (0, ODD, -2), (3, ODD, -2)]:
        a = list(base); a[pos] = val
        assert f(*a) == want, (pos, val)


def test_attn_prefill_validation(lib):
    f = lib.csa2_sparse_attn_prefill
    base = [FAKE, FAKE, FAKE, FAKE, 512, FAKE, 1000, 64, 0.04, FAKE, FAKE, 1 << 40, None]
    for pos, val, want in [(7, 0, -1), (4, -1, -1), (6, -1, -1), (3, None, -1), (0, ODD, -2),
                           (9, ODD, -2), (11, 10, -3), (10, None, -3)]:
        a = list(base); a[pos] = val
        assert f(*a) == want, (pos, val)


def test_prefill_select_validation(lib):
    f = lib.csa2_prefill_select
    base = [FAKE, FAKE, FAKE, 131072, 2, 258048, 4096, 512, FAKE, FAKE, 1 << 40, None]
    for pos, val, want in [(4, 0, -1), (5, -1, -1), (7, 0, -1), (6, 0, -1), (0, ODD, -2),
                           (10, 10, -3), (9, None, -3)]:
        a = list(base); a[pos] = val
        assert f(*a) == want, (pos, val)


def test_replay_select_validation(lib):
    f = lib.csa2_replay_select
    base = [FAKE, FAKE, FAKE, 1 << 20, 1, (1 << 20) - 128, 128, 16384, FAKE, FAKE, 512, FAKE, FAKE,
            1 << 40, None]
    for pos, val, want in [(6, 0, -1), (4, 0, -1), (5, -1, -1), (3, -1, -1), (7, 0, -1),
                           (7, 16385, -1), (10, 0, -1), (10, 16385, -1), (0, None, -1),
                           (8, None, -1), (1, None, -1), (0, ODD, -2), (9, ODD, -2), (11, ODD, -2),
                           (13, 100, -3), (12, None, -3), (3, (1 << 26) + 1, -4)]:
        a = list(base); a[pos] = val
        assert f(*a) == want, (pos, val)
    assert lib.csa2_replay_select_workspace_size(0, 1 << 20, 16384) == 0
    assert lib.csa2_replay_select_workspace_size(128, 1 << 20, 0) == 0
    # the score matrix dominates: T x n_entries fp32
    assert lib.csa2_replay_select_workspace_size(128, 1 << 20, 16384) >= 128 * (1 << 20) * 4
    assert lib.csa2_replay_select_workspace_size(4, 0, 64) > 0


def test_binding_rejects_host_tensors():
    # no CPU fallback: the binding refuses tensors that are not on the GPU before any call
    import torch
    x = torch.zeros((4, 128), dtype=torch.int16)
    y = torch.zeros((4, 512), dtype=torch.int16)
    planes = (torch.zeros((8, 64), dtype=torch.uint8), torch.zeros(8), torch.zeros((8, 256), dtype=torch.uint8),
              torch.zeros((8, 32), dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU"):
        csa2.csa2_kv_append(x, y, torch.arange(4), *planes)
    with pytest.raises(ValueError, match="GPU"):
        csa2.csa2_swa_append(y, torch.arange(4), torch.zeros((4, 128, 512), dtype=torch.uint8))


def test_attention_id_range_check_on_the_host(monkeypatch):
    """The host-side id check (CPU only, no launch): -1 and ids below the row's entry count
    pass; an id at or past it, or below -1, raises before any call."""
    import torch
    n = torch.tensor([10, 3], dtype=torch.int32)
    ok = torch.tensor([[0, 4, 9, -1], [-1, 0, 1, 2]], dtype=torch.int32)
    csa2.check_attention_ids(ok, n)
    for bad, where in [([[0, 4, 10, -1], [-1, 0, 1, 2]], "row 0 position 2"),
                       ([[0, 4, 9, -1], [-1, 0, 3, 2]], "row 1 position 2"),
                       ([[0, -2, 9, -1], [-1, 0, 1, 2]], "row 0 position 1")]:
        with pytest.raises(csa2.Csa2Error, match=where):
            csa2.check_attention_ids(torch.tensor(bad, dtype=torch.int32), n)
    # the attention binding runs it when asked, before anything reaches the library
    monkeypatch.setenv("CSA2_CHECK_IDS", "1")
    bad = torch.tensor([[0, 4, 10, -1], [-1, 0, 1, 2]], dtype=torch.int32)
    with pytest.raises(csa2.Csa2Error, match="outside"):
        csa2.csa2_sparse_attn_decode(None, None, None, None, bad, None, None, None, None, n_entries=n)
