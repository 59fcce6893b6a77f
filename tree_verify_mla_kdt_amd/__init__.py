"""kdt: tree-verify MLA-absorb attention for AMD MI355X (gfx950).

The compute path is the HIP library ``libkdt.so`` behind the C ABI declared in
``include/kdt.h``; ``tree_verify_mla_kdt_amd.kdt`` is its thin ctypes binding.
``synth`` holds the seeded synthetic input generators.
"""
__all__ = ["kdt", "synth"]
