"""CPU pins of the best-first tree-build oracle (no GPU).

The build is pinned by hand-derived trees (tests/golden/tree_build_cases.json,
dyadic log-probabilities so every sum is exact), by brute force (on small
inputs the tree is exactly the q - 1 best paths of the whole candidate tree,
since log-probabilities are <= 0 and a path never outranks its ancestors), by
closed forms (one candidate per position gives a chain, one position a star,
and budgets beyond the candidate tree leave padding), by the lazy-offer variant
a device builder uses (same nodes in the same order, exact ties included, when
ties go by parent creation index and rank), and by the link invariants of the
first-child / next-sibling encoding.  The oracle itself is the plain heap: a
created node pushes all K children, and equal logw pops in push order.
"""
import heapq
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from tree_verify_mla_kdt_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tree_build_cases.json")


def test_golden_hand_derived_trees():
    cases = json.load(open(GOLDEN))["cases"]
    assert len(cases) >= 4
    for c in cases:
        r = oracle.build_tree(np.array([c["topk_tokens"]]), np.array([c["topk_logprobs"]]),
                              [c["root_token"]], c["q"])
        for k in ("parents", "tokens", "depth", "first_child", "next_sibling"):
            assert r[k][0].tolist() == c[k], (c["name"], k)
        want = [float("-inf") if x == "-inf" else x for x in c["logw"]]
        assert r["logw"][0].tolist() == want, c["name"]
        assert int(r["n_nodes"][0]) == c["n_nodes"]


def _paths(tok, lp):
    """Every node of the full candidate tree: (logw, path of ranks)."""
    D, K = tok.shape
    out = []
    for d in range(1, D + 1):
        for ranks in itertools.product(range(K), repeat=d):
            w = 0.0
            for i, j in enumerate(ranks):
                w = w + float(lp[i, j])
            out.append((w, ranks))
    return out


def _rank_path(r, b, node, tok):
    """Ranks along the path root -> node, read back from tokens and depths."""
    path = []
    while node > 0:
        d = int(r["depth"][b, node])
        path.append(int(np.nonzero(tok[b, d - 1] == r["tokens"][b, node])[0][0]))
        node = int(r["parents"][b, node])
    return tuple(reversed(path))


@pytest.mark.parametrize("D,K,q", [(1, 4, 3), (2, 3, 7), (3, 3, 12), (4, 2, 20), (3, 4, 30), (2, 2, 10)])
def test_brute_force_top_paths(D, K, q):
    tok, lp, roots = synth.tree_topk_inputs(6, D, K, seed=D * 10 + K)
    r = oracle.build_tree(tok, lp, roots, q)
    for b in range(tok.shape[0]):
        allp = sorted(_paths(tok[b], lp[b]), key=lambda x: -x[0])
        n = int(r["n_nodes"][b])
        assert n == min(q, 1 + len(allp))
        got = [_rank_path(r, b, i, tok) for i in range(1, n)]
        assert got == [p for _, p in allp[:n - 1]]
        assert np.array_equal(r["logw"][b, 1:n], np.array([w for w, _ in allp[:n - 1]]))


def test_closed_forms():
    tok, lp, roots = synth.tree_topk_inputs(3, 9, 1, seed=5)
    r = oracle.build_tree(tok, lp, roots, 6)                      # K = 1: a chain
    assert np.all(r["parents"] == np.array([-1, 0, 1, 2, 3, 4]))
    assert np.all(r["depth"] == np.arange(6))
    tok, lp, roots = synth.tree_topk_inputs(3, 1, 8, seed=6)
    r = oracle.build_tree(tok, lp, roots, 6)                      # D = 1: a star in rank order
    assert np.all(r["parents"][:, 1:] == 0)
    assert np.array_equal(r["tokens"][:, 1:], tok[:, 0, :5])
    r = oracle.build_tree(tok[:, :, :3], lp[:, :, :3], roots, 6)  # 4 real nodes, 2 padding
    assert np.all(r["n_nodes"] == 4)
    assert np.all(r["tokens"][:, 4:] == -1) and np.all(r["parents"][:, 4:] == 0)
    assert np.all(np.isneginf(r["logw"][:, 4:]))
    assert np.array_equal(r["tokens"][:, 0], roots)


def _lazy_variant(tok, lp, root, q):
    """The lazy form a device builder can use: a created node offers only its
    best child, and a popped candidate offers its next-ranked sibling.  Ties
    are broken by (creation index of the parent, rank), which is the push
    order of the plain heap, so with log-probabilities sorted best first the
    same nodes are created in the same order even under exact ties."""
    D, K = tok.shape
    parents, depth, logw, tokens = [-1], [0], [0.0], [int(root)]
    heap = []
    if D >= 1:
        heapq.heappush(heap, (-(0.0 + float(lp[0, 0])), (0, 0), 1, 0, 0))
    while len(parents) < q and heap:
        negw, _, d, j, par = heapq.heappop(heap)
        node = len(parents)
        parents.append(par)
        depth.append(d)
        logw.append(-negw)
        tokens.append(int(tok[d - 1, j]))
        if j + 1 < K:
            heapq.heappush(heap, (-(logw[par] + float(lp[d - 1, j + 1])), (par, j + 1), d, j + 1, par))
        if d < D:
            heapq.heappush(heap, (-(logw[node] + float(lp[d, 0])), (node, 0), d + 1, 0, node))
    return parents, depth, logw, tokens


def _tie_inputs(B, D, K, seed):
    """Log-probabilities from {-1, -2, -3}, sorted best first: exact in float
    and double, so most logw values tie and the tie rule decides."""
    rng = synth.rng_for(seed)
    lp = -np.sort(rng.integers(1, 4, size=(B, D, K)), axis=-1).astype(np.float32)
    tok = np.tile(np.arange(K, dtype=np.int32), (B, D, 1)) + 100 * np.arange(D, dtype=np.int32)[None, :, None]
    return tok, lp, np.arange(B, dtype=np.int32)


def _check_variant(tok, lp, roots, q):
    r = oracle.build_tree(tok, lp, roots, q)
    for b in range(tok.shape[0]):
        p, d, w, t = _lazy_variant(tok[b], lp[b], roots[b], q)
        n = len(p)
        assert int(r["n_nodes"][b]) == n
        assert r["parents"][b, :n].tolist() == p
        assert r["depth"][b, :n].tolist() == d
        assert r["tokens"][b, :n].tolist() == t
        assert r["logw"][b, :n].tolist() == w


@pytest.mark.parametrize("D,K,q", [(8, 4, 65), (16, 2, 33), (4, 8, 128), (12, 3, 100)])
def test_lazy_offers_equal_plain_heap(D, K, q):
    tok, lp, roots = synth.tree_topk_inputs(8, D, K, seed=100 + D + K)
    _check_variant(tok, lp, roots, q)


@pytest.mark.parametrize("D,K,q", [(6, 4, 128), (12, 3, 65), (3, 8, 100), (2, 2, 7), (5, 5, 40)])
def test_lazy_offers_equal_plain_heap_exact_ties(D, K, q):
    tok, lp, roots = _tie_inputs(12, D, K, 555 + D)
    _check_variant(tok, lp, roots, q)


def test_all_ties_golden_case_differs_from_offer_order():
    """The tie rule matters: breaking ties by the order candidates are offered
    lazily (instead of by push order) gives a different tree on the hand case."""
    c = [c for c in json.load(open(GOLDEN))["cases"] if c["name"].startswith("all ties")][0]
    tok, lp = np.array(c["topk_tokens"]), np.array(c["topk_logprobs"])
    D, K = tok.shape
    parents, logw, heap, order = [-1], [0.0], [], 0
    heapq.heappush(heap, (-float(lp[0, 0]), 0, 1, 0, 0))
    order = 1
    while len(parents) < c["q"] and heap:
        negw, _, d, j, par = heapq.heappop(heap)
        node = len(parents)
        parents.append(par)
        logw.append(-negw)
        if j + 1 < K:
            heapq.heappush(heap, (-(logw[par] + float(lp[d - 1, j + 1])), order, d, j + 1, par))
            order += 1
        if d < D:
            heapq.heappush(heap, (-(logw[node] + float(lp[d, 0])), order, d + 1, 0, node))
            order += 1
    assert parents != c["parents"]
    assert oracle.build_tree(tok[None], lp[None], [c["root_token"]], c["q"])["parents"][0].tolist() == c["parents"]


@pytest.mark.parametrize("D,K,q", [(8, 4, 65), (15, 2, 128), (3, 16, 128), (1, 1, 1), (2, 1, 17)])
def test_link_invariants(D, K, q):
    tok, lp, roots = synth.tree_topk_inputs(5, D, K, seed=200 + D * K)
    r = oracle.build_tree(tok, lp, roots, q)
    for b in range(tok.shape[0]):
        n = int(r["n_nodes"][b])
        par = r["parents"][b]
        assert par[0] == -1 and all(0 <= par[i] < i for i in range(1, q))
        assert all(r["depth"][b, i] == r["depth"][b, par[i]] + 1 for i in range(1, n))
        assert np.all(np.diff(r["logw"][b, :n]) <= 0)                 # created best first
        # first-child / next-sibling lists enumerate each node's children in creation order
        for u in range(n):
            kids, c = [], r["first_child"][b, u]
            while c != -1:
                kids.append(int(c))
                c = r["next_sibling"][b, c]
            assert kids == [i for i in range(1, n) if par[i] == u]
        oracle.build_visibility(par[None, :])                       # a valid tree for the masks
