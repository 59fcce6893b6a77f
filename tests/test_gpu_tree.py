"""GPU parity of the best-first tree builder against the oracle: bit-exact
(node order, tokens, depths, double logw, links), including exact logw ties,
padding, chains, stars and wide candidate lists, and composed with the
visibility build and the greedy accept on the device."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

import oracle
from tree_verify_mla_kdt_amd import kdt, synth
from gpu_util import dev, require_gpu

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tree_build_cases.json")
KEYS = ("parents", "tokens", "depth", "logw", "first_child", "next_sibling", "n_nodes")


def _gpu_tree(tok, lp, roots, q):
    require_gpu()
    r = kdt.build_tree(torch.from_numpy(np.ascontiguousarray(tok, np.int32)).to(dev()),
                       torch.from_numpy(np.ascontiguousarray(lp, np.float32)).to(dev()),
                       torch.from_numpy(np.ascontiguousarray(roots, np.int32)).to(dev()), q)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in r.items()}


def _same(got, ref):
    for k in KEYS:
        assert np.array_equal(got[k], ref[k]), k


@pytest.mark.parametrize("B,D,K,q", [(16, 8, 4, 65), (64, 16, 2, 17), (4, 64, 8, 128), (8, 3, 16, 128),
                                     (2, 1, 1, 1), (5, 2, 3, 40), (3, 127, 1, 128), (3, 1, 64, 65),
                                     (6, 20, 200, 30), (512, 8, 4, 33)])
def test_tree_matches_oracle(B, D, K, q):
    tok, lp, roots = synth.tree_topk_inputs(B, D, K, seed=B + D + K + q)
    _same(_gpu_tree(tok, lp, roots, q), oracle.build_tree(tok, lp, roots, q))


def test_golden_trees_on_device():
    for c in json.load(open(GOLDEN))["cases"]:
        tok = np.array([c["topk_tokens"]], np.int32)
        lp = np.array([c["topk_logprobs"]], np.float32)
        got = _gpu_tree(tok, lp, np.array([c["root_token"]], np.int32), c["q"])
        for k in ("parents", "tokens", "depth", "first_child", "next_sibling"):
            assert got[k][0].tolist() == c[k], (c["name"], k)
        want = [float("-inf") if x == "-inf" else x for x in c["logw"]]
        assert got["logw"][0].tolist() == want
        assert int(got["n_nodes"][0]) == c["n_nodes"]


@pytest.mark.parametrize("D,K,q", [(6, 4, 128), (12, 3, 65), (3, 8, 100)])
def test_exact_ties_follow_push_order(D, K, q):
    """Log-probabilities from {-1, -2, -3} (exact in float and double): most
    logw values tie, so the plain heap's push order (parent creation index,
    then rank) decides nearly every step."""
    rng = synth.rng_for(555 + D)
    B = 12
    lp = -np.sort(rng.integers(1, 4, size=(B, D, K)), axis=-1).astype(np.float32)
    tok = np.tile(np.arange(K, dtype=np.int32), (B, D, 1)) + 100 * np.arange(D, dtype=np.int32)[None, :, None]
    roots = np.arange(B, dtype=np.int32)
    _same(_gpu_tree(tok, lp, roots, q), oracle.build_tree(tok, lp, roots, q))


def test_tree_feeds_visibility_and_accept():
    B, D, K, q = 32, 10, 4, 65
    tok, lp, roots = synth.tree_topk_inputs(B, D, K, seed=77)
    r = kdt.build_tree(torch.from_numpy(tok).to(dev()), torch.from_numpy(lp).to(dev()),
                       torch.from_numpy(roots).to(dev()), q)
    st = torch.zeros(B, dtype=torch.int32, device=dev())
    vis, depth = kdt.build_visibility(r["parents"], seq_status=st)
    pred = torch.from_numpy(synth.accept_inputs(r["parents"].cpu().numpy(), 78)[1]).to(dev())
    acc, n_acc, bonus = kdt.tree_accept(r["parents"], r["tokens"], pred, seq_status=st)
    torch.cuda.synchronize()
    ref = oracle.build_tree(tok, lp, roots, q)
    rvis, rdepth = oracle.build_visibility(ref["parents"])
    assert np.array_equal(vis.cpu().numpy().view(np.uint64), rvis)
    assert np.array_equal(depth.cpu().numpy(), ref["depth"])
    ra, rn, rb = oracle.tree_accept(ref["parents"], ref["tokens"], pred.cpu().numpy())
    assert np.array_equal(acc.cpu().numpy(), ra) and np.array_equal(n_acc.cpu().numpy(), rn)
    assert np.array_equal(bonus.cpu().numpy(), rb)
    assert np.all(st.cpu().numpy() == 0)
