"""The seeded workload generators (mla_inputs): every resident layer of a
workload holds the same sequences at another page layout, and each layer's
block table satisfies the paged calls' contract (checked with the library's
host validator, mla_validate_block_table)."""
import pytest
import torch

from mla_inputs import CONFIGS, make_structure


@pytest.mark.parametrize("name", list(CONFIGS))
def test_layers_share_lengths_and_tables_are_valid(name):
    import mla_latent_kv_06_amd as M
    cfg = CONFIGS[name]
    base = make_structure(cfg, seed=42)
    for layer in (0, 1, 7):
        st = make_structure(cfg, seed=42, layout_seed=42 + layer)
        assert torch.equal(st.seqlens, base.seqlens)
        assert st.num_pages == base.num_pages
        M.mla_validate_block_table(st.block_table, base.seqlens, base.num_pages)
        if layer == 0:
            assert torch.equal(st.block_table, base.block_table)
        used = st.block_table[st.block_table >= 0]
        assert used.unique().numel() == used.numel(), "a page is shared between sequences"
