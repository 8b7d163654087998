"""CPU oracle for the CSA2 compressed-sparse-attention path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
(``compressed_sparse_kv_csa2_amd``) never imports it, and nothing here imports
from the library: the two share no code.  Inputs for both come from ``synth``.

Everything is plain fp64 numpy.  Pins that tie this oracle to the pages, to
number-format specifications and to library routines live in
``tests/test_oracle_pins.py``; no function here is "parity unpinned".
"""
from . import formats, quant_ref
from .csa2_ref import *  # noqa: F401,F403
from .csa2_ref import (D_IDX, D_KV, N_HEADS, POOL, SWA_W, TOPK, attention,  # noqa: F401
                       decode_attention, decode_step_long, decoder_chain, dequant_index_keys,
                       dequant_main, dequant_swa, full_layer, global_kv_bytes,
                       global_kv_bytes_per_token, index_dot_is_exact, index_entry_bytes,
                       index_scores, layer_mode, main_entry_bytes, prefill_chunk, reindex_layer,
                       reuse_layer, reuse_source, topk, visible_entries)
from .quant_ref import (e2m1_encode, e4m3_encode, kv_append, quantize_index_entry,  # noqa: F401
                        quantize_main_entry, swa_append, swa_encode)
