"""CPU oracle (test infrastructure).  Imported only by tests/, the smoke check
and the CPU-baseline leg of the benchmark; never by the library itself."""
from .kdt_oracle import (  # noqa: F401
    words_for, check_parents, ancestor_masks, pack_mask, build_visibility, unpack_row,
    key_mask, verify_attn, verify_attn_rows, attend_chunk, merge_partials, gather_accepted,
    tree_accept, build_tree, rope_neox, tree_positions, absorb_q, absorb_o, append_tree_kv,
)
