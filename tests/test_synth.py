"""The seeded input generators: determinism, shapes and tree structure."""
import numpy as np
import pytest
import torch

from tree_verify_mla_kdt_amd import synth


def test_bf16_rounding_is_rne_and_matches_torch():
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 3.0e-3, 65504.0], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(vals)
    assert bits[0] == 0x3F80
    assert bits[1] == 0x3F80          # tie -> even
    assert bits[2] == 0x3F82          # tie -> even (up)
    rng = synth.rng_for(1)
    x = rng.standard_normal(4096).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(x), ref)
    back = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generate_is_deterministic():
    a = synth.generate(synth.CONFIGS["tiny_fp32"])
    b = synth.generate(synth.CONFIGS["tiny_fp32"])
    for name in ("parents", "prefix_lens", "q_lat", "q_pe", "cache", "accepted", "n_accepted"):
        assert np.array_equal(getattr(a, name), getattr(b, name))


def _depths(p):
    d = np.zeros(len(p), dtype=int)
    for i in range(1, len(p)):
        d[i] = d[p[i]] + 1
    return d


def test_best_first_tree_shape():
    rng = synth.rng_for(2)
    for _ in range(20):
        p = synth.tree_best_first(rng, 65)
        assert p[0] == -1 and all(0 <= p[i] < i for i in range(1, 65))
        assert _depths(p).max() <= 8
        assert np.bincount(p[1:], minlength=65).max() <= 4


def test_deep_chain_tree_shape():
    rng = synth.rng_for(3)
    p = synth.tree_deep_chain(rng, 33)
    d = _depths(p)
    assert list(p[:16]) == [-1] + list(range(15))
    assert d[15] == 15 and d[16:].max() <= 14


def test_small_config_shapes_and_paths():
    cfg = synth.config_variant(synth.CONFIGS["ragged_deep"], B=3, R=16, P=8, H=2,
                               prefix=("uniform", 5, 40))
    inp = synth.generate(cfg)
    assert inp.q_lat.shape == (3, 33, 2, 16) and inp.q_lat.dtype == np.uint16
    assert inp.cache.shape[1] % 64 == 0 and inp.cache.shape[1] >= inp.prefix_lens.max() + 33
    assert inp.n_accepted[0] == 16 and list(inp.accepted[0]) == list(range(16))
    for b in range(3):
        path = inp.accepted[b, :inp.n_accepted[b]]
        assert path[0] == 0
        for k in range(1, len(path)):
            assert inp.parents[b, path[k]] == path[k - 1]


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_config_table(name):
    cfg = synth.CONFIGS[name]
    assert cfg.D == cfg.R + cfg.P
    assert abs(cfg.softmax_scale - (cfg.R + cfg.P) ** -0.5) < 1e-15
