"""Pins for the oracle's verify attention (CPU only).

Each test checks the float64 oracle against something other than itself:
a hand-derived worked example, pure-Python brute force with math.fsum, closed
forms, torch's scaled_dot_product_attention in float64, chain == successive AR
steps, masked-key perturbation, prefix permutation and node relabelling.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tree_verify_mla_kdt_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def split_cache(inp):
    cache = inp.f64("cache")
    R = inp.cfg.R
    return cache[..., :R], cache[..., R:]


def run_oracle(inp, parents=None, prefix_lens=None, scale=None):
    parents = inp.parents if parents is None else parents
    prefix_lens = inp.prefix_lens if prefix_lens is None else prefix_lens
    vis, _ = oracle.build_visibility(parents)
    c_kv, k_pe = split_cache(inp)
    return oracle.verify_attn(inp.f64("q_lat"), inp.f64("q_pe"), c_kv, k_pe, prefix_lens, vis,
                              inp.cfg.softmax_scale if scale is None else scale)


def tiny(**kw):
    cfg = synth.config_variant(synth.CONFIGS["tiny_fp32"], **kw)
    return synth.generate(cfg)


# ---------------------------------------------------------------------------

def test_hand_worked_example():
    doc = json.load(open(os.path.join(GOLDEN, "attention_hand_example.json")))
    assert "Checkpoint" in doc["citation"]
    rows = np.asarray(doc["cache_rows_ckv_kpe"], dtype=np.float64)
    R = doc["R"]
    c_kv = rows[None, :, :R]
    k_pe = rows[None, :, R:]
    q = len(doc["parents"])
    q_lat = np.asarray([[float(x) for x in r] for r in doc["q_lat"]]).reshape(1, q, 1, R)
    q_pe = np.asarray([[float(x) for x in r] for r in doc["q_pe"]]).reshape(1, q, 1, doc["P"])
    vis, _ = oracle.build_visibility(np.asarray([doc["parents"]], dtype=np.int32))
    o, lse = oracle.verify_attn(q_lat, q_pe, c_kv, k_pe, [doc["prefix_len"]], vis, doc["scale"])
    for t in range(q):
        exp_o = [float(Fraction(s)) for s in doc["expected_o"][t]]
        exp_lse = math.log(float(doc["expected_lse"][t].split()[1]))
        assert np.allclose(o[0, t, 0], exp_o, atol=1e-14, rtol=0)
        assert abs(lse[0, t, 0] - exp_lse) < 1e-14


def _brute(inp):
    """Pure-Python loops with math.fsum; masks from an upward parent walk."""
    cfg = inp.cfg
    B, q, H, R, P = cfg.B, cfg.q_len, cfg.H, cfg.R, cfg.P
    ql, qp = inp.f64("q_lat"), inp.f64("q_pe")
    cache = inp.f64("cache")
    scale = cfg.softmax_scale
    o = np.zeros((B, q, H, R))
    lse = np.zeros((B, q, H))
    for b in range(B):
        L = int(inp.prefix_lens[b])
        for t in range(q):
            anc, c = set(), t
            while c != -1:
                anc.add(c)
                c = int(inp.parents[b, c])
            keys = list(range(L)) + [L + j for j in sorted(anc)]
            for h in range(H):
                s = []
                for j in keys:
                    dot = math.fsum(float(ql[b, t, h, r]) * float(cache[b, j, r]) for r in range(R))
                    dot += math.fsum(float(qp[b, t, h, p]) * float(cache[b, j, R + p]) for p in range(P))
                    s.append(scale * dot)
                m = max(s)
                w = [math.exp(x - m) for x in s]
                z = math.fsum(w)
                lse[b, t, h] = m + math.log(z)
                for r in range(R):
                    o[b, t, h, r] = math.fsum(w[k] * float(cache[b, j, r]) for k, j in enumerate(keys)) / z
    return o, lse


def test_brute_force_tiny_config():
    inp = synth.generate(synth.CONFIGS["tiny_fp32"])
    o, lse = run_oracle(inp)
    bo, blse = _brute(inp)
    assert np.max(np.abs(o - bo)) < 1e-12
    assert np.max(np.abs(lse - blse)) < 1e-12


def test_brute_force_ragged_batch_small():
    cfg = synth.Config("small_ragged", 9, "bf16", B=3, H=2, R=16, P=8, q_len=6,
                       prefix=("uniform", 0, 9), tree="uniform")
    inp = synth.generate(cfg)
    o, lse = run_oracle(inp)
    bo, blse = _brute(inp)
    assert np.max(np.abs(o - bo)) < 1e-12
    assert np.max(np.abs(lse - blse)) < 1e-12


def test_closed_form_single_key():
    # L = 0, q = 1: the only key is the token's own row.
    inp = tiny(q_len=1)
    inp.prefix_lens[:] = 0
    o, lse = run_oracle(inp)
    c_kv, k_pe = split_cache(inp)
    ql, qp = inp.f64("q_lat"), inp.f64("q_pe")
    for h in range(inp.cfg.H):
        assert np.array_equal(o[0, 0, h], c_kv[0, 0])
        s = inp.cfg.softmax_scale * (ql[0, 0, h] @ c_kv[0, 0] + qp[0, 0, h] @ k_pe[0, 0])
        assert abs(lse[0, 0, h] - s) < 1e-12


def test_closed_form_zero_queries_is_mean_of_visible_rows():
    inp = tiny()
    inp.q_lat[:] = 0
    inp.q_pe[:] = 0
    o, lse = run_oracle(inp)
    c_kv, _ = split_cache(inp)
    L = int(inp.prefix_lens[0])
    for t in range(inp.cfg.q_len):
        anc, c = [], t
        while c != -1:
            anc.append(c)
            c = int(inp.parents[0, c])
        rows = list(range(L)) + [L + j for j in anc]
        mean = c_kv[0, rows].mean(axis=0)
        for h in range(inp.cfg.H):
            assert np.max(np.abs(o[0, t, h] - mean)) < 1e-13
            assert abs(lse[0, t, h] - math.log(len(rows))) < 1e-13


@pytest.mark.parametrize("L", [0, 5, 32])
def test_chain_equals_torch_sdpa_causal(L):
    inp = tiny(tree="chain")
    inp.prefix_lens[:] = L
    o, _ = run_oracle(inp)
    c_kv, k_pe = split_cache(inp)
    q = inp.cfg.q_len
    N = L + q
    Q = torch.from_numpy(np.concatenate([inp.f64("q_lat"), inp.f64("q_pe")], axis=-1)[0])  # [q, H, D]
    K = torch.from_numpy(np.concatenate([c_kv, k_pe], axis=-1)[0, :N])                     # [N, D]
    V = torch.from_numpy(c_kv[0, :N])
    mask = torch.zeros(q, N, dtype=torch.bool)
    mask[:, :L] = True
    mask[:, L:] = torch.tril(torch.ones(q, q, dtype=torch.bool))
    Qh = Q.permute(1, 0, 2)                                    # [H, q, D]
    Kh = K[None].expand(Qh.shape[0], N, K.shape[1]).contiguous()
    Vh = V[None].expand(Qh.shape[0], N, V.shape[1]).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(Qh, Kh, Vh, attn_mask=mask,
                                                           scale=inp.cfg.softmax_scale)
    assert np.max(np.abs(o[0] - ref.permute(1, 0, 2).numpy())) < 1e-12


def test_chain_equals_successive_ar_steps():
    inp = tiny(tree="chain", q_len=7)
    o, lse = run_oracle(inp)
    c_kv, k_pe = split_cache(inp)
    L = int(inp.prefix_lens[0])
    ql, qp = inp.f64("q_lat"), inp.f64("q_pe")
    one = np.ones((1, 1, 1), dtype=np.uint64)
    for t in range(inp.cfg.q_len):
        # AR step t: q_len 1, prefix L + t; the token's own row is L + t.
        o1, l1 = oracle.verify_attn(ql[:, t:t + 1], qp[:, t:t + 1], c_kv, k_pe, [L + t], one,
                                    inp.cfg.softmax_scale)
        assert np.max(np.abs(o1[0, 0] - o[0, t])) < 1e-12
        assert np.max(np.abs(l1[0, 0] - lse[0, t])) < 1e-12


def test_masked_keys_get_zero_weight_bit_identical():
    inp = tiny(q_len=12)
    o, lse = run_oracle(inp)
    vis, _ = oracle.build_visibility(inp.parents)
    L = int(inp.prefix_lens[0])
    q = inp.cfg.q_len
    rng = synth.rng_for(31)
    pert = inp.cache.copy()
    pert[0, L + q:] = rng.standard_normal(pert[0, L + q:].shape).astype(np.float32) * 50
    inp2 = synth.Inputs(inp.cfg, inp.parents, inp.prefix_lens, inp.q_lat, inp.q_pe, pert,
                        inp.accepted, inp.n_accepted)
    o2, lse2 = run_oracle(inp2)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    # Per token: perturbing a tree row the token cannot see leaves it bit-identical.
    for t in range(q):
        hidden = [j for j in range(q) if not oracle.unpack_row(vis[0, t], q)[j]]
        if not hidden:
            continue
        p3 = inp.cache.copy()
        for j in hidden:
            p3[0, L + j] = 1e3
        inp3 = synth.Inputs(inp.cfg, inp.parents, inp.prefix_lens, inp.q_lat, inp.q_pe, p3,
                            inp.accepted, inp.n_accepted)
        o3, l3 = run_oracle(inp3)
        assert np.array_equal(o3[0, t], o[0, t]) and np.array_equal(l3[0, t], lse[0, t])


def test_prefix_permutation_invariance():
    inp = tiny(q_len=9)
    o, lse = run_oracle(inp)
    L = int(inp.prefix_lens[0])
    perm = synth.rng_for(5).permutation(L)
    c2 = inp.cache.copy()
    c2[0, :L] = inp.cache[0, perm]
    inp2 = synth.Inputs(inp.cfg, inp.parents, inp.prefix_lens, inp.q_lat, inp.q_pe, c2,
                        inp.accepted, inp.n_accepted)
    o2, lse2 = run_oracle(inp2)
    assert np.max(np.abs(o - o2)) < 1e-12
    assert np.max(np.abs(lse - lse2)) < 1e-12


def test_node_relabelling_permutes_output():
    inp = tiny(q_len=11)
    o, lse = run_oracle(inp)
    par = inp.parents[0]
    q = len(par)
    rng = synth.rng_for(77)
    # random topological relabelling pi with pi(0) = 0
    placed, order = {0}, [0]
    while len(order) < q:
        avail = [i for i in range(q) if i not in placed and int(par[i]) in placed]
        pick = avail[int(rng.integers(0, len(avail)))]
        placed.add(pick)
        order.append(pick)
    pi = {old: new for new, old in enumerate(order)}
    new_par = np.full(q, -1, dtype=np.int32)
    for old in range(1, q):
        new_par[pi[old]] = pi[int(par[old])]
    L = int(inp.prefix_lens[0])
    c2 = inp.cache.copy()
    ql2, qp2 = inp.q_lat.copy(), inp.q_pe.copy()
    for old in range(q):
        c2[0, L + pi[old]] = inp.cache[0, L + old]
        ql2[0, pi[old]] = inp.q_lat[0, old]
        qp2[0, pi[old]] = inp.q_pe[0, old]
    inp2 = synth.Inputs(inp.cfg, new_par[None], inp.prefix_lens, ql2, qp2, c2,
                        inp.accepted, inp.n_accepted)
    o2, lse2 = run_oracle(inp2)
    for old in range(q):
        assert np.max(np.abs(o2[0, pi[old]] - o[0, old])) < 1e-12
        assert np.max(np.abs(lse2[0, pi[old]] - lse[0, old])) < 1e-12


def test_rows_variant_matches_full():
    inp = tiny(q_len=9)
    o, lse = run_oracle(inp)
    vis, _ = oracle.build_visibility(inp.parents)
    c_kv, k_pe = split_cache(inp)
    rows = [(0, t, h) for t in range(9) for h in range(4)]
    ro, rl = oracle.verify_attn_rows(inp.f64("q_lat"), inp.f64("q_pe"), c_kv, k_pe,
                                     inp.prefix_lens, vis, inp.cfg.softmax_scale, rows)
    for k, (b, t, h) in enumerate(rows):
        assert np.max(np.abs(ro[k] - o[b, t, h])) < 1e-12
        assert abs(rl[k] - lse[b, t, h]) < 1e-12


def test_capacity_overflow_raises():
    inp = tiny()
    with pytest.raises(ValueError):
        run_oracle(inp, prefix_lens=np.asarray([inp.S_cap], dtype=np.int32))
