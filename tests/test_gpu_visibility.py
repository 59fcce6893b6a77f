"""GPU visibility masks vs the oracle: bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from tree_verify_mla_kdt_amd import kdt, synth
from gpu_util import dev, require_gpu

pytestmark = pytest.mark.gpu


def _run(parents_np):
    require_gpu()
    p = torch.from_numpy(np.ascontiguousarray(parents_np, dtype=np.int32)).to(dev())
    st = torch.zeros(p.shape[0], dtype=torch.int32, device=dev())
    vis, depth = kdt.build_visibility(p, seq_status=st)
    torch.cuda.synchronize()
    return vis.cpu().numpy().view(np.uint64), depth.cpu().numpy(), st.cpu().numpy()


@pytest.mark.parametrize("q", [1, 2, 9, 17, 33, 63, 64, 65, 100, 127, 128])
@pytest.mark.parametrize("kind", ["uniform", "chain", "star", "best_first"])
def test_masks_bit_exact(q, kind):
    if kind == "best_first" and q > 65:
        pytest.skip("best-first trees of depth <= 8 are drawn up to the 65-node budget")
    rng = synth.rng_for(q * 7 + len(kind))
    B = 5
    parents = np.stack([synth.make_tree(rng, kind, q) for _ in range(B)])
    vis, depth, st = _run(parents)
    rv, rd = oracle.build_visibility(parents)
    assert np.array_equal(vis, rv)
    assert np.array_equal(depth, rd)
    assert np.all(st == 0)


def test_config_trees_and_large_batch():
    for name in ("max_budget", "batched", "long_ctx", "ragged_deep"):
        cfg = synth.CONFIGS[name]
        rng = synth.rng_for(cfg.index)
        parents = np.stack([synth.make_tree(rng, cfg.tree, cfg.q_len) for _ in range(max(cfg.B, 3))])
        vis, depth, _ = _run(parents)
        rv, rd = oracle.build_visibility(parents)
        assert np.array_equal(vis, rv) and np.array_equal(depth, rd), name
    rng = synth.rng_for(4242)
    parents = np.stack([synth.tree_uniform(rng, 65) for _ in range(1000)])
    vis, depth, _ = _run(parents)
    rv, rd = oracle.build_visibility(parents)
    assert np.array_equal(vis, rv) and np.array_equal(depth, rd)


def test_invalid_trees_are_flagged_and_bounded():
    good = synth.tree_uniform(synth.rng_for(1), 9)
    bad_root = good.copy(); bad_root[0] = 3
    cyclic = good.copy(); cyclic[4] = 6; cyclic[6] = 4          # a cycle through forward parents
    out_of_range = good.copy(); out_of_range[2] = -7
    parents = np.stack([good, bad_root, cyclic, out_of_range])
    vis, depth, st = _run(parents)
    assert st.tolist() == [0, kdt.KDT_SEQ_BAD_TREE, kdt.KDT_SEQ_BAD_TREE, kdt.KDT_SEQ_BAD_TREE]
    rv, rd = oracle.build_visibility(good[None])
    assert np.array_equal(vis[0], rv[0]) and np.array_equal(depth[0], rd[0])
    # every row of a flagged tree still holds its own bit and nothing at or above q
    for b in range(1, 4):
        for i in range(9):
            w = int(vis[b, i, 0])
            assert (w >> i) & 1 and w >> 9 == 0
    # node 4 of the cyclic tree lost its (forward) parent: it is a root of its own
    assert int(vis[2, 4, 0]) == 1 << 4
