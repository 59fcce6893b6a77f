"""Pins for the oracle's visibility masks (CPU only).

The oracle builds masks by the pages' own rule (parent's mask | own bit).  These
tests check it against hand-derived fixtures, closed forms (chain, star), an
independent brute-force ancestor walk written here, and its error handling.
"""
import json
import os

import numpy as np
import pytest

import oracle
from tree_verify_mla_kdt_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parents_from_spec(spec):
    if isinstance(spec, list):
        return np.asarray(spec, dtype=np.int32)
    if spec == "chain:65":
        return synth.tree_chain(65)
    if spec == "star:65":
        return synth.tree_star(65)
    if spec == "star:65 with parent[64]=63":
        p = synth.tree_star(65)
        p[64] = 63
        return p
    raise AssertionError(spec)


def test_golden_hand_derived_masks():
    doc = json.load(open(os.path.join(GOLDEN, "visibility_cases.json")))
    assert "Milestone" in doc["citation"]
    for case in doc["cases"]:
        parents = _parents_from_spec(case["parents"])
        vis, depth = oracle.build_visibility(parents[None, :])
        if "rows" in case:
            for i, words in enumerate(case["rows"]):
                assert [int(w, 16) for w in words] == [int(x) for x in vis[0, i]], (case["name"], i)
                assert depth[0, i] == case["depth"][i]
        for key, (words, d) in case.get("selected", {}).items():
            i = int(key)
            assert [int(w, 16) for w in words] == [int(x) for x in vis[0, i]], (case["name"], i)
            assert depth[0, i] == d, (case["name"], i)


def _brute_ancestors(parents, i):
    """Walk parent pointers upward from node i (independent of the oracle)."""
    out = set()
    c = int(i)
    steps = 0
    while c != -1:
        out.add(c)
        c = int(parents[c])
        steps += 1
        assert steps <= len(parents)
    return out


@pytest.mark.parametrize("q", [1, 2, 9, 17, 33, 63, 64, 65, 100, 128])
def test_random_trees_match_brute_force_walk(q):
    rng = synth.rng_for(q)
    parents = np.stack([synth.tree_uniform(rng, q) for _ in range(3)])
    vis, depth = oracle.build_visibility(parents)
    W = (q + 63) // 64
    assert vis.shape == (3, q, W) and vis.dtype == np.uint64
    for b in range(3):
        for i in range(q):
            anc = _brute_ancestors(parents[b], i)
            for j in range(W * 64):
                bit = (int(vis[b, i, j // 64]) >> (j % 64)) & 1
                assert bit == (1 if j in anc else 0), (b, i, j)
            assert depth[b, i] == len(anc) - 1


@pytest.mark.parametrize("q", [1, 9, 64, 65, 128])
def test_chain_is_lower_triangle(q):
    vis, depth = oracle.build_visibility(synth.tree_chain(q)[None])
    for i in range(q):
        row = oracle.unpack_row(vis[0, i], q)
        assert row.tolist() == [j <= i for j in range(q)]
        assert depth[0, i] == i


@pytest.mark.parametrize("q", [2, 17, 65, 128])
def test_star_is_diagonal_plus_root(q):
    vis, depth = oracle.build_visibility(synth.tree_star(q)[None])
    for i in range(q):
        row = oracle.unpack_row(vis[0, i], q)
        assert row.tolist() == [(j == i or j == 0) for j in range(q)]
        assert depth[0, i] == (0 if i == 0 else 1)


def test_popcount_is_depth_plus_one_and_padding_zero():
    rng = synth.rng_for(7)
    for q in (65, 97):
        p = synth.tree_best_first(rng, q) if q == 65 else synth.tree_uniform(rng, q)
        vis, depth = oracle.build_visibility(p[None])
        for i in range(q):
            total = sum(bin(int(w)).count("1") for w in vis[0, i])
            assert total == depth[0, i] + 1
            # bits at or above q are zero
            hi = int(vis[0, i, -1]) >> (q - 64 * (vis.shape[2] - 1)) if q % 64 else 0
            assert hi == 0


@pytest.mark.parametrize("bad", [
    [0, 0, 1],          # root parent not -1
    [-1, 1, 0],         # self parent
    [-1, 0, 3, 1],      # forward parent
    [-1, -1, 0],        # second root
    [-1, 0, -5],        # out of range
])
def test_invalid_parents_raise(bad):
    with pytest.raises(ValueError):
        oracle.build_visibility(np.asarray([bad], dtype=np.int32))
