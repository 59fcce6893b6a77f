"""CPU pins of the oracle's steps around the verify: rotary embedding, the
query split + key absorb, the value absorb and the cache append.

Rotary embedding is pinned by its closed form for one pair, by the complex
rotation it is (x1 + i x2 times e^(i angle)), and by its invariants (position
0 is the identity, norms are kept, rotations compose, and the dot product of
a rotated query and key depends only on their position difference).  The
absorbs are pinned by loops with exact summation and by the identities that
motivate them: scores against latents with the absorbed query equal scores
against explicitly up-projected keys, and the absorbed value output equals the
attention average of explicitly up-projected values.
"""
import math

import numpy as np
import pytest

import oracle
from tree_verify_mla_kdt_amd import synth


def test_rope_closed_form_and_complex_rotation():
    for pos in (0, 1, 7, 12345):
        got = oracle.rope_neox([[2.0, -3.0]], [pos], 10000.0)[0]
        assert np.allclose(got, [2 * math.cos(pos) + 3 * math.sin(pos), -3 * math.cos(pos) + 2 * math.sin(pos)],
                           atol=1e-12)
    rng = synth.rng_for(401)
    x = rng.standard_normal((5, 64))
    pos = rng.integers(0, 40000, size=5)
    got = oracle.rope_neox(x, pos, 50000.0)
    for n in range(5):
        for i in range(32):
            ang = pos[n] * 50000.0 ** (-2.0 * i / 64)
            z = complex(x[n, i], x[n, i + 32]) * complex(math.cos(ang), math.sin(ang))
            assert abs(got[n, i] - z.real) < 1e-9 and abs(got[n, i + 32] - z.imag) < 1e-9


def test_rope_invariants():
    rng = synth.rng_for(402)
    x = rng.standard_normal((7, 64))
    k = rng.standard_normal((7, 64))
    assert np.allclose(oracle.rope_neox(x, np.zeros(7), 10000.0), x, atol=0, rtol=0)
    p = rng.integers(0, 5000, size=7)
    rx = oracle.rope_neox(x, p, 10000.0)
    assert np.allclose(np.linalg.norm(rx, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    assert np.allclose(oracle.rope_neox(rx, p + 3, 10000.0), oracle.rope_neox(x, 2 * p + 3, 10000.0), atol=1e-9)
    m, n, s = 100, 37, 2000                      # relative positions only
    d1 = np.sum(oracle.rope_neox(x, np.full(7, m), 1e4) * oracle.rope_neox(k, np.full(7, n), 1e4), axis=-1)
    d2 = np.sum(oracle.rope_neox(x, np.full(7, m + s), 1e4) * oracle.rope_neox(k, np.full(7, n + s), 1e4), axis=-1)
    assert np.allclose(d1, d2, atol=1e-9)


def _small(seed=0, B=2, T=3, H=2, dn=4, P=4, R=6, dv=3):
    inp = synth.absorb_inputs(B, T, H, dn, P, R, dv, seed)
    f = {k: synth.bf16_bits_to_f32(v).astype(np.float64) for k, v in inp.items()}
    return f, (B, T, H, dn, P, R, dv)


def test_absorb_q_loops_and_positions():
    f, (B, T, H, dn, P, R, dv) = _small(1)
    pl = np.array([5, 11])
    depth = np.array([[0, 1, 1], [0, 1, 2]])
    q_lat, q_pe = oracle.absorb_q(f["q"], f["w_kc_t"], pl, depth, dn, 10000.0)
    for b in range(B):
        for t in range(T):
            for h in range(H):
                for r in range(R):
                    want = math.fsum(f["q"][b, t, h, i] * f["w_kc_t"][h, r, i] for i in range(dn))
                    assert abs(q_lat[b, t, h, r] - want) < 1e-12
                rp = oracle.rope_neox(f["q"][b, t, h, dn:], pl[b] + depth[b, t], 10000.0)
                assert np.allclose(q_pe[b, t, h], rp, atol=0, rtol=0)


def test_absorbed_scores_equal_explicit_keys():
    """q_lat . c_kv == q_nope . (W_UK c_kv) with W_UK[h] = w_kc_t[h]^T."""
    f, (B, T, H, dn, P, R, dv) = _small(2, R=16, dn=8)
    c = synth.rng_for(403).standard_normal((9, R))
    q_lat, _ = oracle.absorb_q(f["q"], f["w_kc_t"], np.zeros(B, int), np.zeros((B, T), int), dn, 1e4)
    for h in range(H):
        k_nope = c @ f["w_kc_t"][h]              # [keys, dn]: the un-absorbed keys
        explicit = f["q"][:, :, h, :dn] @ k_nope.T
        absorbed = q_lat[:, :, h, :] @ c.T
        assert np.allclose(explicit, absorbed, atol=1e-10)


def test_absorb_o_loops_and_value_identity():
    f, (B, T, H, dn, P, R, dv) = _small(3)
    o = oracle.absorb_o(f["o_lat"], f["w_vc"])
    for b in range(B):
        for t in range(T):
            for h in range(H):
                for j in range(dv):
                    want = math.fsum(f["w_vc"][h, j, r] * f["o_lat"][b, t, h, r] for r in range(R))
                    assert abs(o[b, t, h, j] - want) < 1e-12
    # attention over latents then absorb == attention over explicit values
    rng = synth.rng_for(404)
    c = rng.standard_normal((11, R))
    p = rng.random(11)
    p /= p.sum()
    lat = (p @ c)[None, None, None, :].repeat(H, axis=2)
    got = oracle.absorb_o(lat, f["w_vc"])[0, 0]
    for h in range(H):
        v = c @ f["w_vc"][h].T                   # explicit values [keys, dv]
        assert np.allclose(got[h], p @ v, atol=1e-12)


def test_append_places_rows_and_rotates_keys():
    f, (B, T, H, dn, P, R, dv) = _small(4)
    S = 24
    cache = synth.rng_for(405).standard_normal((B, S, R + P))
    pl = np.array([3, 17])
    depth = np.array([[0, 1, 2], [0, 1, 1]])
    new = oracle.append_tree_kv(cache, f["c_kv_new"], f["k_rope_new"], pl, depth, 1e4)
    for b in range(B):
        L = pl[b]
        untouched = [i for i in range(S) if not (L <= i < L + T)]
        assert np.array_equal(new[b, untouched], cache[b, untouched])
        assert np.array_equal(new[b, L:L + T, :R], f["c_kv_new"][b])
        for t in range(T):
            assert np.array_equal(new[b, L + t, R:], oracle.rope_neox(f["k_rope_new"][b, t], L + depth[b, t], 1e4))
