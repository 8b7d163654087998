"""Python binding of libcsa2 (the CSA2 hot path for MI355X / gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels behind the
C ABI declared in include/csa2.h.  Tensors are torch device tensors (torch provides
memory and streams); each wrapper checks dtype, shape and contiguity, then passes raw
pointers and the current HIP stream.  There is no fallback: if the shared library is
missing or cannot load, importing the binding's entry points raises.

bf16 values travel as their bit patterns in int16 tensors (or as torch.bfloat16).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "csa2_index_score", "csa2_topk", "csa2_index_topk", "csa2_select_chain",
    "csa2_sparse_attn_decode", "csa2_prefill_chunk", "csa2_topk_workspace_size",
    "csa2_index_topk_workspace_size", "csa2_select_chain_workspace_size", "csa2_attn_workspace_size", "csa2_prefill_workspace_size",
    "topk_workspace", "index_topk_workspace", "select_chain_workspace", "attn_workspace", "prefill_workspace", "lib_path", "load_library",
    "csa2_prefill_select", "csa2_sparse_attn_prefill", "csa2_kv_append", "csa2_swa_append", "CSA2_TOPK_HIST_FUSED", "Csa2Error",
    "csa2_workspace_status", "workspace_status", "PreparedCall", "check_workspace", "csa2_sparse_attn_decode_noalloc",
    "check_attention_ids", "csa2_replay_select", "csa2_replay_select_workspace_size",
    "replay_select_workspace",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libcsa2.so")
CSA2_TOPK_HIST_FUSED = 1
_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F32 = ctypes.c_float
_U32 = ctypes.c_uint32

_SIGS = {
    "csa2_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "csa2_version": (ctypes.c_int, []),
    "csa2_index_score": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I32, _P, _P, _SZ, _P]),
    "csa2_topk_workspace_size": (_SZ, [_I32, _I32, _I32]),
    "csa2_topk": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _I32, _P, _P, _U32, _P, _SZ, _P]),
    "csa2_index_topk_workspace_size": (_SZ, [_I32, _I32, _I32]),
    "csa2_index_topk": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _SZ,
                                       _P]),
    "csa2_select_chain_workspace_size": (_SZ, [_I32, _I32, _I32]),
    "csa2_select_chain": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _I32, _P, _P,
                                         _I32, _P, _P, _P, _SZ, _P]),
    "csa2_workspace_status": (ctypes.c_int, [_P, _P, _P]),
    "csa2_replay_select_workspace_size": (_SZ, [_I32, _I32, _I32]),
    "csa2_replay_select": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I64, _I32, _I32, _P, _P, _I32, _P,
                                          _P, _SZ, _P]),
    "csa2_attn_workspace_size": (_SZ, [_I32, _I32]),
    "csa2_sparse_attn_decode": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _P, _P, _F32, _I32, _P, _P,
                                               _SZ, _P]),
    "csa2_sparse_attn_decode_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _P, _P, _F32, _I32,
                                                       _P, _P]),
    "csa2_attn_noalloc_max_bytes": (_SZ, []),
    "csa2_prefill_workspace_size": (_SZ, [_I32, _I32, _I32]),
    "csa2_prefill_chunk": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I64, _I32, _I32, _P,
                                          _F32, _P, _P, _P, _SZ, _P]),
    "csa2_prefill_select": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I64, _I32, _I32, _P, _P, _SZ,
                                           _P]),
    "csa2_sparse_attn_prefill": (ctypes.c_int, [_P, _P, _P, _P, _I32, _P, _I64, _I32, _F32, _P, _P,
                                                _SZ, _P]),
    "csa2_kv_append": (ctypes.c_int, [_P, _P, _P, _I32, _P, _P, _P, _P, _I64, _P, _P]),
    "csa2_swa_append": (ctypes.c_int, [_P, _P, _I32, _P, _P]),
}


class Csa2Error(RuntimeError):
    pass


def load_library():
    """Load libcsa2.so (built by compressed_sparse_kv_csa2_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise Csa2Error(f"{lib_path} is missing: build it with "
                        "`python -m compressed_sparse_kv_csa2_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(lib_path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        msg = load_library().csa2_status_string(status).decode()
        raise Csa2Error(f"csa2 call failed: {msg} ({status})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class PreparedCall:
    """A C-ABI call whose arguments were checked and marshalled once: calling it issues the
    same call again (same buffers, same stream), for steps that repeat their launches.  The
    buffers' contents may change between calls; their addresses and shapes may not."""

    __slots__ = ("_fn", "_args", "_pre")

    def __init__(self, fn, args, pre=None):
        self._fn, self._args, self._pre = fn, args, pre

    def __call__(self):
        if self._pre is not None:
            self._pre()
        _check(self._fn(*self._args))


def _issue(fn, args, prepare, pre=None):
    call = PreparedCall(fn, args, pre)
    if prepare:
        return call
    call()
    return None


def _need(t: torch.Tensor, name: str, dtypes, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None:
        want = tuple(shape)
        if len(want) != t.dim() or any(w is not None and w != s for w, s in zip(want, t.shape)):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want}")


_BF16 = (torch.int16, torch.bfloat16)
_U8 = (torch.uint8,)


# ----------------------------------------------------------------------------- sizes
def csa2_topk_workspace_size(batch: int, n_cols: int, k: int) -> int:
    return int(load_library().csa2_topk_workspace_size(batch, n_cols, k))


def csa2_index_topk_workspace_size(batch: int, n_cols: int, k: int) -> int:
    return int(load_library().csa2_index_topk_workspace_size(batch, n_cols, k))


def csa2_select_chain_workspace_size(batch: int, n_cols: int, pool_k: int) -> int:
    return int(load_library().csa2_select_chain_workspace_size(batch, n_cols, pool_k))


def csa2_replay_select_workspace_size(T: int, n_entries: int, pool_k: int) -> int:
    return int(load_library().csa2_replay_select_workspace_size(T, n_entries, pool_k))


def csa2_attn_workspace_size(batch: int, k: int) -> int:
    return int(load_library().csa2_attn_workspace_size(batch, k))


def csa2_prefill_workspace_size(T: int, n_entries: int, k: int) -> int:
    return int(load_library().csa2_prefill_workspace_size(T, n_entries, k))


def _zeros(nbytes: int, device) -> torch.Tensor:
    return torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=device)


def topk_workspace(batch, n_cols, k, device="cuda"):
    """Zero-filled workspace for csa2_topk (and the fused histogram of csa2_index_score)."""
    return _zeros(csa2_topk_workspace_size(batch, n_cols, k), device)


def index_topk_workspace(batch, n_cols, k, device="cuda"):
    """Zero-filled workspace for csa2_index_topk (its first int32 is the status word)."""
    return _zeros(csa2_index_topk_workspace_size(batch, n_cols, k), device)


def select_chain_workspace(batch, n_cols, pool_k, device="cuda"):
    """Zero-filled workspace for csa2_select_chain (its first int32 is the status word)."""
    return _zeros(csa2_select_chain_workspace_size(batch, n_cols, pool_k), device)


def replay_select_workspace(T, n_entries, pool_k, device="cuda"):
    """Zero-filled workspace for csa2_replay_select (its first int32 is the status word)."""
    return _zeros(csa2_replay_select_workspace_size(T, n_entries, pool_k), device)


def csa2_workspace_status(workspace, stream=None):
    """(error bits, rows re-scanned) from the status block of a csa2_index_topk /
    csa2_select_chain / csa2_replay_select workspace; synchronizes the stream."""
    _need(workspace, "workspace", _U8)
    out = (ctypes.c_uint32 * 2)()
    _check(load_library().csa2_workspace_status(_ptr(workspace), ctypes.cast(out, ctypes.c_void_p),
                                                _stream(stream)))
    return int(out[0]), int(out[1])


def workspace_status(workspace, stream=None) -> int:
    """The sticky error bits of a selection workspace (0 after correct calls)."""
    return csa2_workspace_status(workspace, stream)[0]


def check_workspace(workspace, stream=None):
    """Raises Csa2Error when a selection workspace reports an error; the workspace is then
    zero-filled so that it can serve the next call (that call's results were undefined)."""
    bits = workspace_status(workspace, stream)
    if bits:
        workspace.zero_()
        raise Csa2Error(f"selection workspace reports error bits {bits:#x}: results of the calls "
                        "since the last check are undefined (workspace re-zeroed)")


def attn_workspace(batch, k, device="cuda"):
    return _zeros(csa2_attn_workspace_size(batch, k), device)


def prefill_workspace(T, n_entries, k, device="cuda"):
    return _zeros(csa2_prefill_workspace_size(T, n_entries, k), device)


# ----------------------------------------------------------------------------- calls
def csa2_index_score(q_idx, idx_codes, idx_scale, seq_base, n_valid, scores, cand=None,
                     topk_ws=None, stream=None):
    """Scores [B, n_cols] of entries seq_base[b] + (cand[b][c] or c) against q_idx[b]."""
    B, n_cols = scores.shape
    _need(q_idx, "q_idx", _BF16, (B, 128))
    _need(idx_codes, "idx_codes", _U8, (None, 64))
    _need(idx_scale, "idx_scale", (torch.float32,), (idx_codes.shape[0],))
    _need(seq_base, "seq_base", (torch.int64,), (B,))
    _need(n_valid, "n_valid", (torch.int32,), (B,))
    _need(scores, "scores", (torch.float32,), (B, n_cols))
    if cand is not None:
        _need(cand, "cand", (torch.int32,), (B, n_cols))
    if topk_ws is not None:
        _need(topk_ws, "topk_ws", _U8)
    lib = load_library()
    _check(lib.csa2_index_score(_ptr(q_idx), _ptr(idx_codes), _ptr(idx_scale), _ptr(seq_base),
                                _ptr(n_valid), _ptr(cand), B, n_cols, _ptr(scores), _ptr(topk_ws),
                                0 if topk_ws is None else topk_ws.numel(), _stream(stream)))


def csa2_topk(scores, n_valid, k, idx_out, score_out=None, cand=None, hist_fused=False,
              workspace=None, stream=None):
    """idx_out [B, k]: the k best columns of each row, ascending entry ids, -1 padded."""
    B, n_cols = scores.shape
    _need(scores, "scores", (torch.float32,), (B, n_cols))
    _need(n_valid, "n_valid", (torch.int32,), (B,))
    _need(idx_out, "idx_out", (torch.int32,), (B, k))
    if score_out is not None:
        _need(score_out, "score_out", (torch.float32,), (B, k))
    if cand is not None:
        _need(cand, "cand", (torch.int32,), (B, n_cols))
    if workspace is not None:
        _need(workspace, "workspace", _U8)
    lib = load_library()
    _check(lib.csa2_topk(_ptr(scores), B, n_cols, _ptr(n_valid), _ptr(cand), k, _ptr(idx_out),
                         _ptr(score_out), CSA2_TOPK_HIST_FUSED if hist_fused else 0, _ptr(workspace),
                         0 if workspace is None else workspace.numel(), _stream(stream)))


def csa2_index_topk(q_idx, idx_codes, idx_scale, seq_base, n_valid, k, idx_out, workspace,
                    n_cols, score_out=None, cand=None, stream=None, prepare=False):
    """csa2_index_score + csa2_topk in one call: idx_out [B, k] of the n_cols columns.
    prepare=True returns the checked call as a PreparedCall instead of issuing it."""
    B = q_idx.shape[0]
    _need(q_idx, "q_idx", _BF16, (B, 128))
    _need(idx_codes, "idx_codes", _U8, (None, 64))
    _need(idx_scale, "idx_scale", (torch.float32,), (idx_codes.shape[0],))
    _need(seq_base, "seq_base", (torch.int64,), (B,))
    _need(n_valid, "n_valid", (torch.int32,), (B,))
    _need(idx_out, "idx_out", (torch.int32,), (B, k))
    if score_out is not None:
        _need(score_out, "score_out", (torch.float32,), (B, k))
    if cand is not None:
        _need(cand, "cand", (torch.int32,), (B, n_cols))
    _need(workspace, "workspace", _U8)
    lib = load_library()
    return _issue(lib.csa2_index_topk,
                  (_ptr(q_idx), _ptr(idx_codes), _ptr(idx_scale), _ptr(seq_base), _ptr(n_valid),
                   _ptr(cand), B, n_cols, k, _ptr(idx_out), _ptr(score_out), _ptr(workspace),
                   workspace.numel(), _stream(stream)), prepare)


def csa2_select_chain(q_full, idx_codes, idx_scale, seq_base, n_valid, n_cols, pool_out, workspace,
                      k=512, pool_score_out=None, own_out=None, q_re=None, re_out=None,
                      re_score_out=None, stream=None, prepare=False):
    """Full scan -> pool_out [B, pool_k]; own_out [B, k] (the Full layer's top-k inside the
    pool); re_out [R, B, k] for the Reindex queries q_re [R, B, 128].  prepare=True returns
    the checked call as a PreparedCall instead of issuing it."""
    B, pool_k = pool_out.shape
    _need(q_full, "q_full", _BF16, (B, 128))
    _need(idx_codes, "idx_codes", _U8, (None, 64))
    _need(idx_scale, "idx_scale", (torch.float32,), (idx_codes.shape[0],))
    _need(seq_base, "seq_base", (torch.int64,), (B,))
    _need(n_valid, "n_valid", (torch.int32,), (B,))
    _need(pool_out, "pool_out", (torch.int32,), (B, pool_k))
    if pool_score_out is not None:
        _need(pool_score_out, "pool_score_out", (torch.float32,), (B, pool_k))
    if own_out is not None:
        _need(own_out, "own_out", (torch.int32,), (B, k))
    n_re = 0
    if q_re is not None:
        n_re = q_re.shape[0]
        _need(q_re, "q_re", _BF16, (n_re, B, 128))
        _need(re_out, "re_out", (torch.int32,), (n_re, B, k))
        if re_score_out is not None:
            _need(re_score_out, "re_score_out", (torch.float32,), (n_re, B, k))
    _need(workspace, "workspace", _U8)
    lib = load_library()
    return _issue(lib.csa2_select_chain,
                  (_ptr(q_full), _ptr(idx_codes), _ptr(idx_scale), _ptr(seq_base), _ptr(n_valid), B,
                   n_cols, pool_k, _ptr(pool_out), _ptr(pool_score_out), k, _ptr(own_out),
                   _ptr(q_re), n_re, _ptr(re_out), _ptr(re_score_out), _ptr(workspace),
                   workspace.numel(), _stream(stream)), prepare)


def csa2_replay_select(q_idx, idx_codes, idx_scale, n_entries, ratio, pos0, pool_out, workspace,
                       k=512, own_out=None, pool_n_out=None, stream=None):
    """Per query t of q_idx [T, 128] (position pos0 + t): pool_out [T, pool_k], the pool of its
    best visible entries; own_out [T, k] (optional), its top-k inside the pool; pool_n_out
    [T] (optional), the valid entries of each pool."""
    T, pool_k = pool_out.shape
    _need(q_idx, "q_idx", _BF16, (T, 128))
    _need(idx_codes, "idx_codes", _U8, (None, 64))
    _need(idx_scale, "idx_scale", (torch.float32,), (idx_codes.shape[0],))
    if idx_codes.shape[0] < n_entries:
        raise ValueError("fewer cache entries than n_entries")
    _need(pool_out, "pool_out", (torch.int32,), (T, pool_k))
    if own_out is not None:
        _need(own_out, "own_out", (torch.int32,), (T, k))
    if pool_n_out is not None:
        _need(pool_n_out, "pool_n_out", (torch.int32,), (T,))
    _need(workspace, "workspace", _U8)
    _check(load_library().csa2_replay_select(_ptr(q_idx), _ptr(idx_codes), _ptr(idx_scale),
                                             int(n_entries), int(ratio), int(pos0), T, pool_k,
                                             _ptr(pool_out), _ptr(pool_n_out), int(k), _ptr(own_out),
                                             _ptr(workspace), workspace.numel(), _stream(stream)))


def check_attention_ids(idx, n_entries):
    """Host-side range check of attention lists: every id of row b must be -1 (skip) or in
    [0, n_entries[b]).  idx: int32 [B, k] and n_entries: [B] (either device), copied to the
    host; raises Csa2Error naming the first bad row and id.  The library cannot check this
    itself: its attention call takes no per-sequence entry count, so an id out of range
    would read outside the sequence's entries."""
    import numpy as np
    ids = idx.detach().to("cpu").numpy()
    n = np.asarray(n_entries.detach().to("cpu").numpy() if hasattr(n_entries, "detach") else n_entries,
                   dtype=np.int64).reshape(-1)
    if ids.ndim != 2 or n.shape[0] != ids.shape[0]:
        raise Csa2Error(f"id check: idx {tuple(ids.shape)} and n_entries {tuple(n.shape)} disagree")
    bad = (ids < -1) | (ids >= n[:, None])
    if bad.any():
        b, j = map(int, np.argwhere(bad)[0])
        raise Csa2Error(f"attention list row {b} position {j}: id {int(ids[b, j])} outside "
                        f"[-1, {int(n[b])})")


def _ids_checked() -> bool:
    return os.environ.get("CSA2_CHECK_IDS", "") not in ("", "0")


def csa2_sparse_attn_decode(q, kv_codes, kv_scale, seq_base, idx, swa, swa_len, out, workspace,
                            softmax_scale=512 ** -0.5, stream=None, n_entries=None, prepare=False):
    """out [B, 16, 512] f32: one softmax over the selected entries and the window rows.
    When n_entries (int32 [B]) is given and the environment sets CSA2_CHECK_IDS=1, the list
    is range-checked on the host before each issue (check_attention_ids).  prepare=True
    returns the checked call as a PreparedCall instead of issuing it."""
    pre = None
    if idx is not None and n_entries is not None and _ids_checked():
        if prepare:
            pre = lambda: check_attention_ids(idx, n_entries)
        else:
            check_attention_ids(idx, n_entries)
    B = q.shape[0]
    _need(q, "q", _BF16, (B, 16, 512))
    _need(kv_codes, "kv_codes", _U8, (None, 256))
    _need(kv_scale, "kv_scale", _U8, (kv_codes.shape[0], 32))
    _need(seq_base, "seq_base", (torch.int64,), (B,))
    k = 0
    if idx is not None:
        _need(idx, "idx", (torch.int32,), (B, None))
        k = idx.shape[1]
    _need(swa, "swa", _U8, (B, 128, 512))
    _need(swa_len, "swa_len", (torch.int32,), (B,))
    _need(out, "out", (torch.float32,), (B, 16, 512))
    _need(workspace, "workspace", _U8)
    lib = load_library()
    return _issue(lib.csa2_sparse_attn_decode,
                  (_ptr(q), _ptr(kv_codes), _ptr(kv_scale), _ptr(seq_base),
                   _ptr(idx) if k > 0 else None, k, _ptr(swa), _ptr(swa_len), float(softmax_scale), B,
                   _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)), prepare, pre)


def csa2_sparse_attn_decode_noalloc(q, kv_codes, kv_scale, seq_base, idx, swa, swa_len, out,
                                    softmax_scale=512 ** -0.5, stream=None):
    """csa2_sparse_attn_decode with the library's static scratch instead of a workspace."""
    B = q.shape[0]
    _need(q, "q", _BF16, (B, 16, 512))
    _need(kv_codes, "kv_codes", _U8, (None, 256))
    _need(kv_scale, "kv_scale", _U8, (kv_codes.shape[0], 32))
    _need(seq_base, "seq_base", (torch.int64,), (B,))
    k = 0
    if idx is not None:
        _need(idx, "idx", (torch.int32,), (B, None))
        k = idx.shape[1]
    _need(swa, "swa", _U8, (B, 128, 512))
    _need(swa_len, "swa_len", (torch.int32,), (B,))
    _need(out, "out", (torch.float32,), (B, 16, 512))
    lib = load_library()
    _check(lib.csa2_sparse_attn_decode_noalloc(_ptr(q), _ptr(kv_codes), _ptr(kv_scale), _ptr(seq_base),
                                               _ptr(idx) if k > 0 else None, k, _ptr(swa), _ptr(swa_len),
                                               float(softmax_scale), B, _ptr(out), _stream(stream)))


def csa2_prefill_chunk(q_idx, q, idx_codes, idx_scale, kv_codes, kv_scale, n_entries, ratio, pos0,
                       k, swa, idx_out, out, workspace, softmax_scale=512 ** -0.5, stream=None):
    """T queries at positions pos0..pos0+T-1: causal scoring, per-query top-k, attention."""
    T = q_idx.shape[0]
    _need(q_idx, "q_idx", _BF16, (T, 128))
    _need(q, "q", _BF16, (T, 16, 512))
    _need(idx_codes, "idx_codes", _U8, (None, 64))
    _need(idx_scale, "idx_scale", (torch.float32,), (idx_codes.shape[0],))
    _need(kv_codes, "kv_codes", _U8, (None, 256))
    _need(kv_scale, "kv_scale", _U8, (kv_codes.shape[0], 32))
    if idx_codes.shape[0] < n_entries or kv_codes.shape[0] < n_entries:
        raise ValueError("fewer cache entries than n_entries")
    _need(swa, "swa", _U8, (T + 127, 512))
    _need(idx_out, "idx_out", (torch.int32,), (T, k))
    _need(out, "out", (torch.float32,), (T, 16, 512))
    _need(workspace, "workspace", _U8)
    lib = load_library()
    _check(lib.csa2_prefill_chunk(_ptr(q_idx), _ptr(q), _ptr(idx_codes), _ptr(idx_scale),
                                  _ptr(kv_codes), _ptr(kv_scale), int(n_entries), int(ratio),
                                  int(pos0), T, int(k), _ptr(swa), float(softmax_scale),
                                  _ptr(idx_out), _ptr(out), _ptr(workspace), workspace.numel(),
                                  _stream(stream)))


def csa2_kv_append(x_idx, x_kv, dst, idx_codes, idx_scale, kv_codes, kv_scale, bad=None,
                   stream=None):
    """Quantise rows of x_idx [n,128] / x_kv [n,512] (bf16) into entries dst [n] (int64) of the
    four planes; rows whose dst is outside the planes are skipped and counted into bad [1]."""
    n = x_idx.shape[0]
    _need(x_idx, "x_idx", _BF16, (n, 128))
    _need(x_kv, "x_kv", _BF16, (n, 512))
    _need(dst, "dst", (torch.int64,), (n,))
    _need(idx_codes, "idx_codes", _U8, (None, 64))
    cap = idx_codes.shape[0]
    _need(idx_scale, "idx_scale", (torch.float32,), (cap,))
    _need(kv_codes, "kv_codes", _U8, (cap, 256))
    _need(kv_scale, "kv_scale", _U8, (cap, 32))
    if bad is not None:
        _need(bad, "bad", (torch.int32,), (1,))
    _check(load_library().csa2_kv_append(_ptr(x_idx), _ptr(x_kv), _ptr(dst), n, _ptr(idx_codes),
                                         _ptr(idx_scale), _ptr(kv_codes), _ptr(kv_scale), cap,
                                         _ptr(bad), _stream(stream)))


def csa2_swa_append(x, pos, swa, stream=None):
    """swa[b][pos[b] % 128] = E4M3(x[b]) for every sequence with pos[b] >= 0."""
    B = x.shape[0]
    _need(x, "x", _BF16, (B, 512))
    _need(pos, "pos", (torch.int64,), (B,))
    _need(swa, "swa", _U8, (B, 128, 512))
    _check(load_library().csa2_swa_append(_ptr(x), _ptr(pos), B, _ptr(swa), _stream(stream)))


def csa2_sparse_attn_prefill(q, kv_codes, kv_scale, idx, swa, pos0, out, workspace,
                             softmax_scale=512 ** -0.5, stream=None):
    """out [T, 16, 512]: query t (position pos0 + t) over its list idx[t] (entry ids from 0;
    None for none) and its causal window from swa [T + 127, 512] (row r = position pos0-127+r).
    workspace: attn_workspace(T, k)."""
    T = q.shape[0]
    _need(q, "q", _BF16, (T, 16, 512))
    _need(kv_codes, "kv_codes", _U8, (None, 256))
    _need(kv_scale, "kv_scale", _U8, (kv_codes.shape[0], 32))
    k = 0
    if idx is not None:
        _need(idx, "idx", (torch.int32,), (T, None))
        k = idx.shape[1]
    _need(swa, "swa", _U8, (T + 127, 512))
    _need(out, "out", (torch.float32,), (T, 16, 512))
    _need(workspace, "workspace", _U8)
    _check(load_library().csa2_sparse_attn_prefill(_ptr(q), _ptr(kv_codes), _ptr(kv_scale),
                                                   _ptr(idx) if k > 0 else None, k, _ptr(swa),
                                                   int(pos0), T, float(softmax_scale), _ptr(out),
                                                   _ptr(workspace), workspace.numel(),
                                                   _stream(stream)))


def csa2_prefill_select(q_idx, idx_codes, idx_scale, n_entries, ratio, pos0, k, idx_out, workspace,
                        stream=None):
    """idx_out [T, k]: the per-query top-k of csa2_prefill_chunk, without its attention."""
    T = q_idx.shape[0]
    _need(q_idx, "q_idx", _BF16, (T, 128))
    _need(idx_codes, "idx_codes", _U8, (None, 64))
    _need(idx_scale, "idx_scale", (torch.float32,), (idx_codes.shape[0],))
    if idx_codes.shape[0] < n_entries:
        raise ValueError("fewer cache entries than n_entries")
    _need(idx_out, "idx_out", (torch.int32,), (T, k))
    _need(workspace, "workspace", _U8)
    _check(load_library().csa2_prefill_select(_ptr(q_idx), _ptr(idx_codes), _ptr(idx_scale),
                                              int(n_entries), int(ratio), int(pos0), T, int(k),
                                              _ptr(idx_out), _ptr(workspace), workspace.numel(),
                                              _stream(stream)))
