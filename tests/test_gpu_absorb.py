"""GPU parity of the steps around the verify (query split + key absorb +
rotary embedding, value absorb, tree-token cache append) against the oracle,
and of the whole chain absorb_q -> cache append -> verify -> absorb_o."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tree_verify_mla_kdt_amd import kdt, synth
from gpu_util import check_close, dev, require_gpu

pytestmark = pytest.mark.gpu
THETA = 50000.0


def _bf(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev()).view(torch.bfloat16)


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _f(a):
    return synth.bf16_bits_to_f32(a).astype(np.float64)


@pytest.mark.parametrize("B,T,H,dn,P,R,big", [(2, 9, 16, 128, 64, 512, False), (1, 65, 16, 128, 64, 512, True),
                                              (3, 5, 4, 64, 32, 256, False), (2, 17, 8, 256, 64, 512, True),
                                              (1, 3, 2, 32, 16, 128, False)])
def test_absorb_q_matches_oracle(B, T, H, dn, P, R, big):
    require_gpu()
    inp = synth.absorb_inputs(B, T, H, dn, P, R, 128, seed=B + T + H + dn)
    rng = synth.rng_for(700 + T)
    pl = rng.integers(0, 200000 if big else 3000, size=B).astype(np.int32)
    depth = rng.integers(0, T, size=(B, T)).astype(np.int32)
    q = _bf(inp["q"])
    if big:                                     # a strided view: each head row padded by 16 values
        pad = torch.zeros((B, T, H, dn + P + 16), dtype=torch.bfloat16, device=dev())
        pad[..., :dn + P] = q
        q = pad[..., :dn + P]
    q_lat, q_pe = kdt.absorb_q(q, _bf(inp["w_kc_t"]), torch.from_numpy(pl).to(dev()),
                               torch.from_numpy(depth).to(dev()), dn, THETA)
    torch.cuda.synchronize()
    r_lat, r_pe = oracle.absorb_q(_f(inp["q"]), _f(inp["w_kc_t"]), pl, depth, dn, THETA)
    check_close("bf16", _f64(q_lat), r_lat, np.zeros(1), np.zeros(1), "q_lat")
    check_close("bf16", _f64(q_pe), r_pe, np.zeros(1), np.zeros(1), "q_pe")


@pytest.mark.parametrize("B,T,H,R,dv", [(2, 9, 16, 512, 128), (1, 65, 16, 512, 128), (3, 7, 4, 256, 64),
                                        (2, 3, 2, 128, 128)])
def test_absorb_o_matches_oracle(B, T, H, R, dv):
    require_gpu()
    inp = synth.absorb_inputs(B, T, H, 128, 64, R, dv, seed=R + dv + T)
    o = kdt.absorb_o(_bf(inp["o_lat"]), _bf(inp["w_vc"]))
    torch.cuda.synchronize()
    check_close("bf16", _f64(o), oracle.absorb_o(_f(inp["o_lat"]), _f(inp["w_vc"])), np.zeros(1), np.zeros(1),
                "o")


def test_append_writes_rows_and_flags_bad_lengths():
    require_gpu()
    B, T, R, P, S = 3, 9, 512, 64, 256
    inp = synth.absorb_inputs(B, T, 4, 128, P, R, 128, seed=9)
    rng = synth.rng_for(701)
    cache_np = synth.f32_to_bf16_bits(rng.standard_normal((B, S, R + P)).astype(np.float32))
    pl = np.array([10, 200, 250], np.int32)     # the last one does not fit: 250 + 9 > 256
    depth = rng.integers(0, T, size=(B, T)).astype(np.int32)
    cache = _bf(cache_np)
    st = torch.zeros(B, dtype=torch.int32, device=dev())
    kdt.append_tree_kv(cache, _bf(inp["c_kv_new"]), _bf(inp["k_rope_new"]), torch.from_numpy(pl).to(dev()),
                       torch.from_numpy(depth).to(dev()), THETA, seq_status=st)
    torch.cuda.synchronize()
    got = cache.cpu().view(torch.int16).numpy().view(np.uint16)
    assert st.cpu().tolist() == [0, 0, kdt.KDT_SEQ_BAD_LEN]
    ref = oracle.append_tree_kv(_f(cache_np[:2]), _f(inp["c_kv_new"][:2]), _f(inp["k_rope_new"][:2]), pl[:2],
                                depth[:2], THETA)                                 # the sequences that fit
    for b in range(2):
        L = pl[b]
        keep = [i for i in range(S) if not (L <= i < L + T)]
        assert np.array_equal(got[b, keep], cache_np[b, keep])                  # other rows untouched
        assert np.array_equal(got[b, L:L + T, :R], inp["c_kv_new"][b])          # latents copied exactly
        check_close("bf16", _f(got[b, L:L + T, R:]), ref[b, L:L + T, R:], np.zeros(1), np.zeros(1), "k_pe")
    assert np.array_equal(got[2], cache_np[2])                                   # skipped sequence


def test_chain_absorb_append_verify_absorb():
    """absorb_q -> append -> verify -> absorb_o on the device against the same
    chain in the oracle (every step from the same bf16 inputs)."""
    require_gpu()
    B, q, H, dn, P, R, dv = 2, 17, 16, 128, 64, 512, 128
    cfg = synth.Config("chain", 90, "bf16", B=B, H=H, R=R, P=P, q_len=q, prefix=("uniform", 100, 900),
                       tree="best_first")
    base = synth.generate(cfg)
    inp = synth.absorb_inputs(B, q, H, dn, P, R, dv, seed=90)
    parents = torch.from_numpy(base.parents).to(dev())
    pl = torch.from_numpy(base.prefix_lens).to(dev())
    vis, depth = kdt.build_visibility(parents)
    q_lat, q_pe = kdt.absorb_q(_bf(inp["q"]), _bf(inp["w_kc_t"]), pl, depth, dn, THETA)
    cache = _bf(base.cache)
    kdt.append_tree_kv(cache, _bf(inp["c_kv_new"]), _bf(inp["k_rope_new"]), pl, depth, THETA)
    o_lat, lse = kdt.verify_attn(q_lat, q_pe, cache[..., :R], cache[..., R:], pl, vis, cfg.softmax_scale,
                                 max_prefix_len=int(base.prefix_lens.max()))
    o = kdt.absorb_o(o_lat, _bf(inp["w_vc"]))
    torch.cuda.synchronize()
    # oracle chain, on the bf16 values the device used at each boundary
    depth_np = depth.cpu().numpy()
    r_lat, r_pe = oracle.absorb_q(_f(inp["q"]), _f(inp["w_kc_t"]), base.prefix_lens, depth_np, dn, THETA)
    check_close("bf16", _f64(q_lat), r_lat, np.zeros(1), np.zeros(1), "q_lat")
    r_cache = oracle.append_tree_kv(_f(base.cache), _f(inp["c_kv_new"]), _f(inp["k_rope_new"]),
                                    base.prefix_lens, depth_np, THETA)
    rvis, _ = oracle.build_visibility(base.parents)
    ro_lat, rlse = oracle.verify_attn(_f64(q_lat), _f64(q_pe), _f64(cache[..., :R]), _f64(cache[..., R:]),
                                      base.prefix_lens, rvis, cfg.softmax_scale)
    check_close("bf16", _f64(o_lat), ro_lat, lse.cpu().numpy(), rlse, "verify")
    check_close("bf16", _f64(o), oracle.absorb_o(_f64(o_lat), _f(inp["w_vc"])), np.zeros(1), np.zeros(1), "o")
    # the appended rotary keys themselves
    cache_np = _f64(cache)
    for b in range(B):
        L = base.prefix_lens[b]
        check_close("bf16", cache_np[b, L:L + q, R:], r_cache[b, L:L + q, R:], np.zeros(1), np.zeros(1), "k_pe")
