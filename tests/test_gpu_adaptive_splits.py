"""GPU: adaptive splits (the library's choice of split size).  Every sequence
is cut into splits of about as many key tiles as one of the longest
sequence's, so short and long sequences give the split workgroups the same
work; with the sum of the prefix lengths as a hint the plan sizes the launch
for the sequences it really has.  Checked against the float64 oracle at full
size and on extreme mixes of lengths, the partials of every split against the
oracle on the split's own keys, and the stage-by-stage route (partials, then
the merge over all splits) bit-exact against kdt_verify_attn.  (schedule 1:
splits, where the library could choose the balanced schedule.)"""
import numpy as np
import pytest
import torch

import oracle
from tree_verify_mla_kdt_amd import kdt, synth
from gpu_util import GpuInputs, check_close, oracle_by_seq, require_gpu, to_f64

pytestmark = pytest.mark.gpu


def _plan(g, **kw):
    kw.setdefault("schedule", 1)
    d, _, _ = kdt._verify_prepare(g.q_lat, g.q_pe, g.c_kv, g.k_pe, g.prefix_lens, None, g.cfg.softmax_scale,
                                  g.max_prefix_len, None, None, None, 0, parents=g.parents, **kw)
    return kdt.verify_plan(d)


def _run(g, **kw):
    kw.setdefault("schedule", 1)
    out, lse = kdt.verify_attn(g.q_lat, g.q_pe, g.c_kv, g.k_pe, g.prefix_lens, None, g.cfg.softmax_scale,
                               max_prefix_len=g.max_prefix_len, parents=g.parents, **kw)
    torch.cuda.synchronize()
    return out, lse


def _split_tiles(n_keys, split, max_splits, tiles_max):
    """The adaptive split rule, restated (tiles of 32 keys)."""
    T = -(-n_keys // 32)
    want = -(-T * max_splits // tiles_max)
    tps = -(-T // want)
    return min(split * tps, T), min((split + 1) * tps, T), -(-T // tps)


@pytest.mark.parametrize("layout", [0, 1, 4])
def test_ragged_deep_with_length_hint(layout):
    require_gpu()
    inp = synth.generate(synth.CONFIGS["ragged_deep"])
    g = GpuInputs(inp)
    hint = int(inp.prefix_lens.sum())
    p = _plan(g, total_prefix_len=hint, layout=layout)
    assert p.tiles_max > 0 and p.max_splits > 1
    o, l = _run(g, total_prefix_len=hint, layout=layout)
    ro, rl = oracle_by_seq(inp)
    check_close("bf16", to_f64(o), ro, l.cpu().numpy().astype(np.float64), rl, f"ragged_deep layout {p.layout}")


@pytest.mark.parametrize("lens", [[0, 5, 31, 32, 33, 4000, 6000, 6031],
                                  [6000, 1, 1, 1, 1, 1, 1, 1],
                                  [17, 900, 2, 4096, 64, 3000, 128, 96]])
def test_extreme_length_mixes(lens):
    require_gpu()
    cfg = synth.Config("adaptive_mix", 61, "bf16", B=len(lens), H=16, R=512, P=64, q_len=17,
                       prefix=("fixed", max(lens)), tree="uniform")
    inp = synth.generate(cfg)
    inp.prefix_lens[:] = np.asarray(lens, np.int32)          # (the cache holds N(0,1) rows everywhere)
    g = GpuInputs(inp)
    for hint in (0, int(sum(lens))):
        for layout in (1, 2, 4):
            o, l = _run(g, total_prefix_len=hint, layout=layout)
            ro, rl = oracle_by_seq(inp)
            check_close("bf16", to_f64(o), ro, l.cpu().numpy().astype(np.float64), rl, f"mix {lens} {hint} {layout}")


def test_partials_follow_the_adaptive_rule_and_merge_over_all_splits():
    """Each split's partial equals the oracle on the split's own key tiles;
    unused splits carry lse = -inf; merging all max_splits splits gives
    kdt_verify_attn's output bit for bit."""
    require_gpu()
    cfg = synth.Config("adaptive_parts", 62, "bf16", B=4, H=16, R=512, P=64, q_len=9,
                       prefix=("fixed", 3000), tree="uniform")
    inp = synth.generate(cfg)
    inp.prefix_lens[:] = np.asarray([3000, 1500, 700, 40], np.int32)
    g = GpuInputs(inp)
    hint = int(inp.prefix_lens.sum())
    part_o, part_lse, p = kdt.verify_partials(g.q_lat, g.q_pe, g.c_kv, g.k_pe, g.prefix_lens, None,
                                              cfg.softmax_scale, max_prefix_len=g.max_prefix_len,
                                              parents=g.parents, total_prefix_len=hint, layout=1, schedule=1)
    torch.cuda.synchronize()
    assert p.tiles_max > 0
    S, M = p.max_splits, p.rows
    po = kdt.untile_partials(part_o, M).float().cpu().numpy().astype(np.float64)
    pl = part_lse.cpu().numpy().astype(np.float64)
    vis, _ = oracle.build_visibility(inp.parents)
    cache = inp.f64("cache")
    ql, qp = inp.f64("q_lat"), inp.f64("q_pe")
    q, H = cfg.q_len, cfg.H
    for b in range(cfg.B):
        L = int(inp.prefix_lens[b])
        N = L + q
        for s in range(S):
            t0, t1, ns = _split_tiles(N, s, S, p.tiles_max)
            if s >= ns:
                assert np.all(np.isneginf(pl[b, s])), (b, s)
                continue
            for t in range(q):
                mask_full = oracle.key_mask(L, vis[b, t], q)
                for h in (0, H - 1):
                    mask = np.zeros(N, bool)
                    mask[t0 * 32:min(N, t1 * 32)] = True
                    mask &= mask_full
                    ro, rl = oracle.attend_chunk(ql[b, t, h], qp[b, t, h], cache[b, :N, :cfg.R], cache[b, :N, cfg.R:],
                                                 mask, cfg.softmax_scale)
                    m = t * H + h
                    if np.isneginf(rl):
                        assert np.isneginf(pl[b, s, m])
                        continue
                    assert abs(pl[b, s, m] - rl) < 2e-2
                    assert np.max(np.abs(po[b, s, m] - ro)) < 2e-2
    out_m, lse_m = kdt.merge_partials(part_o, part_lse, q, H, torch.bfloat16)
    out_d, lse_d = _run(g, total_prefix_len=hint, layout=1)
    torch.cuda.synchronize()
    assert torch.equal(lse_m, lse_d)
    assert torch.equal(out_m, out_d)


def test_fused_merge_with_adaptive_splits():
    require_gpu()
    # (lengths the fused merge can take: every split workgroup resident at once)
    cfg = synth.Config("adaptive_fused", 63, "bf16", B=6, H=16, R=512, P=64, q_len=17,
                       prefix=("uniform", 100, 1200), tree="uniform")
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    hint = int(inp.prefix_lens.sum())
    p = _plan(g, total_prefix_len=hint, layout=1, merge_mode=1)
    assert p.tiles_max > 0 and p.fused_merge == 1
    ws = torch.zeros(p.workspace_bytes, dtype=torch.uint8, device=g.q_lat.device)
    o1, l1 = _run(g, total_prefix_len=hint, layout=1, merge_mode=1, workspace=ws)
    o2, l2 = _run(g, total_prefix_len=hint, layout=1)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
