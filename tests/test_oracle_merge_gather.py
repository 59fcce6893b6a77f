"""Pins for the oracle's partial merge and accepted-path gather (CPU only)."""
import math

import numpy as np
import pytest

import oracle
from tree_verify_mla_kdt_amd import synth


def _one_row(seed=3, N=40, R=16, P=4):
    rng = synth.rng_for(seed)
    return (rng.standard_normal(R), rng.standard_normal(P), rng.standard_normal((N, R)),
            rng.standard_normal((N, P)))


@pytest.mark.parametrize("cuts", [[0, 40], [0, 10, 40], [0, 0, 13, 13, 27, 40], [0, 1, 2, 3, 40]])
def test_any_partition_merges_to_unsplit(cuts):
    ql, qp, ck, kp = _one_row()
    mask = np.ones(40, dtype=bool)
    mask[[5, 17, 33]] = False
    o_full, l_full = oracle.attend_chunk(ql, qp, ck, kp, mask, 0.3)
    parts = [oracle.attend_chunk(ql, qp, ck[a:b], kp[a:b], mask[a:b], 0.3)
             for a, b in zip(cuts[:-1], cuts[1:])]
    o, l = oracle.merge_partials([p[0] for p in parts], [p[1] for p in parts])
    assert np.max(np.abs(o - o_full)) < 1e-12 and abs(l - l_full) < 1e-12


def test_merge_is_associative_and_handles_empty_chunks():
    ql, qp, ck, kp = _one_row(N=30)
    mask = np.ones(30, dtype=bool)
    a = oracle.attend_chunk(ql, qp, ck[:7], kp[:7], mask[:7], 0.5)
    b = oracle.attend_chunk(ql, qp, ck[7:19], kp[7:19], mask[7:19], 0.5)
    c = oracle.attend_chunk(ql, qp, ck[19:], kp[19:], mask[19:], 0.5)
    e = (np.zeros(16), -np.inf)
    ab = oracle.merge_partials([a[0], b[0]], [a[1], b[1]])
    left = oracle.merge_partials([ab[0], c[0]], [ab[1], c[1]])
    bc = oracle.merge_partials([b[0], c[0]], [b[1], c[1]])
    right = oracle.merge_partials([a[0], bc[0], e[0]], [a[1], bc[1], e[1]])
    assert np.max(np.abs(left[0] - right[0])) < 1e-12 and abs(left[1] - right[1]) < 1e-12
    # all chunks empty: lse -inf, output zero
    o, l = oracle.merge_partials([e[0], e[0]], [e[1], e[1]])
    assert l == -np.inf and np.all(o == 0)


def test_merge_closed_form_equal_weights():
    o1, o2 = np.array([1.0, 2.0]), np.array([3.0, -2.0])
    o, l = oracle.merge_partials([o1, o2], [0.7, 0.7])
    assert np.allclose(o, [2.0, 0.0], atol=1e-15) and abs(l - (0.7 + math.log(2))) < 1e-15
    o, l = oracle.merge_partials([o1, o2], [math.log(3.0), 0.0])   # weights 3:1
    assert np.allclose(o, [1.5, 1.0], atol=1e-15) and abs(l - math.log(4.0)) < 1e-15


# ---------------------------------------------------------------------------

def test_gather_matches_fancy_indexing_and_leaves_other_rows():
    inp = synth.generate(synth.CONFIGS["tiny_fp32"])
    cfg = synth.config_variant(synth.CONFIGS["tiny_fp32"], B=5, q_len=9)
    inp = synth.generate(cfg)
    new = oracle.gather_accepted(inp.cache, inp.prefix_lens, inp.accepted, inp.n_accepted)
    for b in range(cfg.B):
        L, n = int(inp.prefix_lens[b]), int(inp.n_accepted[b])
        ref = inp.cache[b].copy()
        ref[L:L + n] = inp.cache[b][L + inp.accepted[b, :n]]
        assert np.array_equal(new[b], ref)
        untouched = np.r_[0:L, L + n:inp.S_cap]
        assert np.array_equal(new[b, untouched], inp.cache[b, untouched])


def test_gather_overlapping_in_place_reads_before_writes():
    cache = np.arange(10, dtype=np.float32).reshape(1, 10, 1) * np.ones((1, 1, 3), np.float32)
    # acc = [0, 2, 3]: row 1 <- row 2 while row 2 <- row 3 (a sequential
    # in-place loop in the wrong order would copy row 3 into row 1)
    new = oracle.gather_accepted(cache, [4], np.asarray([[0, 2, 3]]), [3])
    assert new[0, 4:7, 0].tolist() == [4.0, 6.0, 7.0]
    assert new[0, 7:, 0].tolist() == [7.0, 8.0, 9.0]
    # a rotation: every destination is also a source; only read-before-write
    # semantics give the rotated rows (a sequential loop would repeat row 6)
    new = oracle.gather_accepted(cache, [4], np.asarray([[2, 0, 1]]), [3])
    assert new[0, 4:7, 0].tolist() == [6.0, 4.0, 5.0]
    assert new[0, :4, 0].tolist() == [0.0, 1.0, 2.0, 3.0]


def test_gather_then_ar_step_equals_tree_row():
    """Greedy-exact in miniature: after gathering the path to node t, one AR
    step (q_len 1) over prefix L + depth(t) gives verify row t."""
    cfg = synth.config_variant(synth.CONFIGS["tiny_fp32"], q_len=9)
    inp = synth.generate(cfg)
    vis, depth = oracle.build_visibility(inp.parents)
    R = cfg.R
    cache = inp.f64("cache")
    ql, qp = inp.f64("q_lat"), inp.f64("q_pe")
    o, lse = oracle.verify_attn(ql, qp, cache[..., :R], cache[..., R:], inp.prefix_lens, vis,
                                cfg.softmax_scale)
    L = int(inp.prefix_lens[0])
    one = np.ones((1, 1, 1), dtype=np.uint64)
    for t in range(cfg.q_len):
        path = synth.path_to(inp.parents[0], t)
        g = oracle.gather_accepted(cache, inp.prefix_lens, path[None], [len(path)])
        d = int(depth[0, t])
        o1, l1 = oracle.verify_attn(ql[:, t:t + 1], qp[:, t:t + 1], g[..., :R], g[..., R:],
                                    [L + d], one, cfg.softmax_scale)
        assert np.max(np.abs(o1[0, 0] - o[0, t])) < 1e-12
        assert np.max(np.abs(l1[0, 0] - lse[0, t])) < 1e-12
