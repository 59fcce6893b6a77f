"""Pins for the oracle's greedy tree accept (CPU only).

The accepted path is fixed by three properties, which together define it
uniquely: it starts at the root and every step goes from a node to a child
whose token is the node's prediction (greedy consistency); every step takes
the lowest-index such child (tie rule); it ends at a node none of whose
children carries its prediction (maximality).  The tests check those
properties on random trees, the hand-derived golden cases, and closed forms
(chain with every prediction followed; no prediction followed; q = 1)."""
import json
import os

import numpy as np
import pytest

import oracle
from tree_verify_mla_kdt_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "accept_cases.json")


def test_golden_hand_derived_cases():
    for c in json.load(open(GOLDEN))["cases"]:
        q = len(c["parents"])
        acc, n, bonus = oracle.tree_accept(np.array([c["parents"]]), np.array([c["tokens"]]),
                                           np.array([c["pred"]]))
        assert n[0] == c["n_accepted"], c["name"]
        assert acc[0, :n[0]].tolist() == c["accepted"], c["name"]
        assert np.all(acc[0, n[0]:] == -1) and acc.shape == (1, q)
        assert bonus[0] == c["bonus"], c["name"]


def _check_properties(parents, tokens, pred, acc, n, bonus):
    q = len(parents)
    path = acc[:n].tolist()
    assert path[0] == 0 and 1 <= n <= q
    for a, c in zip(path[:-1], path[1:]):
        assert parents[c] == a                                # a root path
        assert tokens[c] == pred[a]                            # greedy consistency
        assert not any(parents[s] == a and tokens[s] == pred[a] for s in range(1, c))   # lowest index
    last = path[-1]
    assert not any(parents[s] == last and tokens[s] == pred[last] for s in range(1, q))  # maximality
    assert bonus == pred[last]


@pytest.mark.parametrize("shape,q", [("uniform", 17), ("best_first", 65), ("deep_chain", 33), ("uniform", 128)])
def test_random_trees_satisfy_the_defining_properties(shape, q):
    rng = synth.rng_for(31 + q)
    parents = np.stack([synth.make_tree(rng, shape, q) for _ in range(24)]).astype(np.int32)
    tokens, pred = synth.accept_inputs(parents, seed=q)
    acc, n, bonus = oracle.tree_accept(parents, tokens, pred)
    lengths = set()
    for b in range(parents.shape[0]):
        _check_properties(parents[b], tokens[b], pred[b], acc[b], int(n[b]), int(bonus[b]))
        lengths.add(int(n[b]))
    assert len(lengths) > 2            # the generator gives varied acceptance lengths


def test_chain_with_every_prediction_followed_accepts_everything():
    q = 40
    parents = synth.tree_chain(q)[None].astype(np.int32)
    tokens = np.arange(q, dtype=np.int32)[None] + 100
    pred = np.arange(1, q + 1, dtype=np.int32)[None] + 100
    acc, n, bonus = oracle.tree_accept(parents, tokens, pred)
    assert n[0] == q and acc[0].tolist() == list(range(q)) and bonus[0] == q + 100


def test_no_prediction_followed_accepts_only_the_root():
    rng = synth.rng_for(77)
    parents = np.stack([synth.make_tree(rng, "uniform", 30) for _ in range(5)]).astype(np.int32)
    tokens = np.zeros_like(parents)
    pred = np.ones_like(parents)                       # no child ever carries token 1
    acc, n, bonus = oracle.tree_accept(parents, tokens, pred)
    assert np.all(n == 1) and np.all(acc[:, 0] == 0) and np.all(acc[:, 1:] == -1) and np.all(bonus == 1)


def test_invalid_parents_raise():
    with pytest.raises(ValueError):
        oracle.tree_accept(np.array([[-1, 0, 5]]), np.zeros((1, 3), np.int32), np.zeros((1, 3), np.int32))
