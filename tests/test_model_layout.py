"""The decode runner's layer layout equals the oracle's reading of the pages' layout
("DeepSeek-V4.1 模型结构（0）：一张图看懂 DeepSeek-V4.1-Flash", Q&A on how the 40 layers are
laid out), which tests/golden/layer_layout_pages.txt pins.  Runs without a GPU."""
from compressed_sparse_kv_csa2_amd import model
import oracle


def test_layer_layout_matches_oracle():
    for l in range(model.N_LAYERS):
        mode = oracle.layer_mode(l)
        if l in model.WINDOW_ONLY:
            assert mode == "swa"
        elif l in model.SELECTING:
            assert mode in ("full", "reindex") and model.list_source(l) == l
            assert (l in model.REINDEX) == (mode == "reindex")
        else:
            assert mode == "reuse" and model.list_source(l) == oracle.reuse_source(l)
