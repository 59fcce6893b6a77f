"""GPU: the balanced schedule (stream-K style).  Row-tile groups of every
sequence are streams of key tiles laid end to end and cut into equal ranges,
one per gang of workgroups, so a workgroup may finish one sequence's keys
and go on to the next.  Checked against the float64 oracle at full size
(every row of ragged_deep, sampled rows of long_ctx), on extreme length mixes
where one workgroup walks many short sequences, with invalid lengths, wrong
length hints, gang sizes that leave the last row-tile group short, both
layouts, float32 inputs and AR decoding; each range's partial against the
oracle on that range's own keys (the balance rule restated below); and the
stage-by-stage route (partials, then the public merge over all slots)
bit-exact against kdt_verify_attn's gated merge."""
import numpy as np
import pytest
import torch

import oracle
from tree_verify_mla_kdt_amd import kdt, synth
from gpu_util import (GpuInputs, check_close, oracle_by_seq, oracle_rows, require_gpu, sample_rows, to_f64)

pytestmark = pytest.mark.gpu


def _plan(g, **kw):
    d, _, _ = kdt._verify_prepare(g.q_lat, g.q_pe, g.c_kv, g.k_pe, g.prefix_lens, None, g.cfg.softmax_scale,
                                  g.max_prefix_len, None, None, None, 0, parents=g.parents, **kw)
    return kdt.verify_plan(d)


def _run(g, max_prefix_len=None, **kw):
    require_gpu()
    out, lse = kdt.verify_attn(g.q_lat, g.q_pe, g.c_kv, g.k_pe, g.prefix_lens, None, g.cfg.softmax_scale,
                               max_prefix_len=g.max_prefix_len if max_prefix_len is None else max_prefix_len,
                               parents=g.parents, **kw)
    torch.cuda.synchronize()
    return out, lse


def _check_full(inp, out, lse, what):
    ro, rl = oracle_by_seq(inp)
    check_close(inp.cfg.dtype, to_f64(out), ro, lse.cpu().numpy().astype(np.float64), rl, what)


def balanced_ranges(lens, q, n_rt, gang, gangs, max_splits, max_prefix_len, capacity, piece_units):
    """The balance rule, restated: [(b, grp, split, first tile, end tile)] for
    every piece (end tiles clipped to the stream)."""
    ceil = lambda x, y: -(-x // y)
    bad = [L < 0 or L > max_prefix_len or L + q > capacity for L in lens]
    T = [1 if bd else ceil(L + q, 32) for L, bd in zip(lens, bad)]
    c = [0 if bd else piece_units for bd in bad]            # start-up units before the key tiles
    n_grp = ceil(n_rt, gang)
    U = n_grp * (sum(T) + sum(c))
    tmax = max([t for t, bd in zip(T, bad) if not bd] + [1])
    A = max(ceil(U, gangs), ceil(tmax, max_splits - 1), 1)
    out, st = [], 0
    for b, t in enumerate(T):
        for grp in range(n_grp):
            r = st + c[b]                                  # first key-tile unit
            for j in range(r // A, (r + t - 1) // A + 1):
                s0, s1 = max(r, j * A), min(r + t, (j + 1) * A)
                out.append((b, grp, j - r // A, s0 - r, s1 - r))
            st += c[b] + t
    return out, A


@pytest.mark.parametrize("layout,gang", [(0, 0), (1, 1), (1, 5), (1, 2), (2, 4), (2, 9)])
def test_ragged_deep_full(layout, gang):
    inp = synth.generate(synth.CONFIGS["ragged_deep"])
    g = GpuInputs(inp)
    hint = int(inp.prefix_lens.sum())
    kw = dict(total_prefix_len=hint, layout=layout, schedule=2, gang_size=gang)
    p = _plan(g, **kw)
    assert p.gang_size > 0 and (gang == 0 or p.gang_size == gang)
    o, l = _run(g, **kw)
    _check_full(inp, o, l, f"ragged_deep balanced layout {p.layout} gang {p.gang_size}")


@pytest.mark.parametrize("gang", [0, 3, 11, 33])
def test_long_ctx_sampled(gang):
    inp = synth.generate(synth.CONFIGS["long_ctx"])
    g = GpuInputs(inp)
    kw = dict(total_prefix_len=int(inp.prefix_lens.sum()), layout=1, schedule=2, gang_size=gang)
    o, l = _run(g, **kw)
    rows = sample_rows(inp, 48, seed=gang)
    ro, rl = oracle_rows(inp, rows)
    go = np.stack([to_f64(o[b, t, h]) for (b, t, h) in rows])
    gl = np.asarray([float(l[b, t, h]) for (b, t, h) in rows])
    check_close("bf16", go, ro, gl, rl, f"long_ctx balanced gang {gang}")
    assert torch.isfinite(o.float()).all() and torch.isfinite(l).all()


@pytest.mark.parametrize("lens", [[0, 5, 31, 32, 33, 4000, 6000, 6031],
                                  [6000] + [1] * 39,
                                  [3, 0, 7, 1, 64, 2, 96, 5, 31, 9, 0, 4, 2, 1, 3, 200],
                                  [17, 900, 2, 4096, 64, 3000, 128, 96]])
@pytest.mark.parametrize("layout", [1, 2])
def test_extreme_length_mixes(lens, layout):
    """Many short sequences: one gang's range covers several whole streams,
    so its workgroups walk from sequence to sequence."""
    cfg = synth.Config("balanced_mix", 71, "bf16", B=len(lens), H=16, R=512, P=64, q_len=17,
                       prefix=("fixed", max(lens)), tree="uniform")
    inp = synth.generate(cfg)
    inp.prefix_lens[:] = np.asarray(lens, np.int32)
    g = GpuInputs(inp)
    for hint in (0, int(sum(lens)), 1, 50 * int(sum(lens)) + 10):     # unknown, right, far too small, far too large
        o, l = _run(g, total_prefix_len=hint, layout=layout, schedule=2)
        _check_full(inp, o, l, f"mix {lens[:6]} hint {hint} layout {layout}")


def test_invalid_lengths_are_skipped_and_flagged():
    cfg = synth.Config("balanced_bad", 72, "bf16", B=6, H=16, R=512, P=64, q_len=17,
                       prefix=("fixed", 700), tree="uniform")
    inp = synth.generate(cfg)
    inp.prefix_lens[:] = np.asarray([700, 650, 300, 20, 500, 0], np.int32)
    g = GpuInputs(inp)
    g.prefix_lens[1] = 900            # beyond the bound passed below
    g.prefix_lens[3] = -5
    st = torch.zeros(6, dtype=torch.int32, device=g.q_lat.device)
    for layout in (1, 2):
        st.zero_()
        o, l = _run(g, max_prefix_len=700, seq_status=st, total_prefix_len=2000, layout=layout, schedule=2,
                    gang_size=2)
        flags = st.cpu().tolist()
        assert flags == [0, kdt.KDT_SEQ_BAD_LEN, 0, kdt.KDT_SEQ_BAD_LEN, 0, 0], flags
        for b in (1, 3):
            assert torch.all(o[b] == 0) and torch.all(torch.isneginf(l[b]))
        keep = [0, 2, 4, 5]
        sub = synth.Inputs(synth.config_variant(cfg, B=len(keep)), inp.parents[keep], inp.prefix_lens[keep],
                           inp.q_lat[keep], inp.q_pe[keep], inp.cache[keep], inp.accepted[keep],
                           inp.n_accepted[keep])
        _check_full(sub, o[keep], l[keep], f"valid sequences, layout {layout}")


def test_float32_tiny_and_small_rank():
    inp = synth.generate(synth.CONFIGS["tiny_fp32"])
    g = GpuInputs(inp)
    o, l = _run(g, schedule=2)
    _check_full(inp, o, l, "tiny fp32 balanced")
    cfg = synth.Config("balanced_r64", 73, "bf16", B=5, H=8, R=64, P=16, q_len=9,
                       prefix=("uniform", 10, 900), tree="uniform")
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    for layout in (1, 2):
        o, l = _run(g, schedule=2, layout=layout, total_prefix_len=int(inp.prefix_lens.sum()))
        _check_full(inp, o, l, f"R=64 balanced layout {layout}")


@pytest.mark.parametrize("name", ["max_budget", "long_ctx"])
def test_ar_q1(name):
    cfg = synth.config_variant(synth.CONFIGS[name], q_len=1)
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    o, l = _run(g, schedule=2, total_prefix_len=int(inp.prefix_lens.sum()))
    _check_full(inp, o, l, f"{name} q=1 balanced")


@pytest.mark.parametrize("layout,gang", [(1, 2), (2, 3)])
def test_partials_follow_the_balance_rule_and_merge_over_all_slots(layout, gang):
    """Each range's partial equals the oracle on that range's own key tiles;
    the other slots carry lse = -inf; the public merge over every slot gives
    kdt_verify_attn's output (gated merge) bit for bit."""
    cfg = synth.Config("balanced_parts", 74, "bf16", B=5, H=16, R=512, P=64, q_len=9,
                       prefix=("fixed", 3000), tree="uniform")
    inp = synth.generate(cfg)
    inp.prefix_lens[:] = np.asarray([3000, 40, 1500, 700, 0], np.int32)
    g = GpuInputs(inp)
    hint = int(inp.prefix_lens.sum())
    kw = dict(total_prefix_len=hint, layout=layout, schedule=2, gang_size=gang)
    part_o, part_lse, p = kdt.verify_partials(g.q_lat, g.q_pe, g.c_kv, g.k_pe, g.prefix_lens, None,
                                              cfg.softmax_scale, max_prefix_len=g.max_prefix_len,
                                              parents=g.parents, **kw)
    torch.cuda.synchronize()
    assert p.gang_size == gang
    S, M = p.max_splits, p.rows
    q, H = cfg.q_len, cfg.H
    BM = 128 if p.layout == 1 else 64
    n_rt = -(-M // BM)
    assert p.piece_units > 0
    pieces, _ = balanced_ranges([int(x) for x in inp.prefix_lens], q, n_rt, p.gang_size, p.gangs, S,
                                g.max_prefix_len, g.c_kv.shape[1], p.piece_units)
    po = kdt.untile_partials(part_o, M).float().cpu().numpy().astype(np.float64)
    pl = part_lse.cpu().numpy().astype(np.float64)
    vis, _ = oracle.build_visibility(inp.parents)
    cache = inp.f64("cache")
    ql, qp = inp.f64("q_lat"), inp.f64("q_pe")
    used = np.zeros((cfg.B, S, M), bool)
    for (b, grp, split, t0, t1) in pieces:
        assert split < S
        L = int(inp.prefix_lens[b])
        N = L + q
        rows = [m for rt in range(grp * p.gang_size, min(n_rt, (grp + 1) * p.gang_size))
                for m in range(rt * BM, min(M, (rt + 1) * BM))]
        used[b, split, rows] = True
        for m in rows[::7] + rows[-1:]:
            t, h = divmod(m, H)
            mask = np.zeros(N, bool)
            mask[t0 * 32:min(N, t1 * 32)] = True
            mask &= oracle.key_mask(L, vis[b, t], q)
            ro, rl = oracle.attend_chunk(ql[b, t, h], qp[b, t, h], cache[b, :N, :cfg.R], cache[b, :N, cfg.R:],
                                         mask, cfg.softmax_scale)
            if np.isneginf(rl):
                assert np.isneginf(pl[b, split, m])
                continue
            assert abs(pl[b, split, m] - rl) < 2e-2, (b, split, m)
            assert np.max(np.abs(po[b, split, m] - ro)) < 2e-2, (b, split, m)
    assert np.all(np.isneginf(pl[~used]))
    out_m, lse_m = kdt.merge_partials(part_o, part_lse, q, H, torch.bfloat16)
    out_d, lse_d = _run(g, **kw)
    assert torch.equal(lse_m, lse_d)
    assert torch.equal(out_m, out_d)


def test_noalloc_with_balanced_schedule():
    cfg = synth.Config("balanced_noalloc", 75, "bf16", B=8, H=16, R=512, P=64, q_len=17,
                       prefix=("uniform", 100, 2500), tree="uniform")
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    hint = int(inp.prefix_lens.sum())
    p = _plan(g, total_prefix_len=hint, schedule=2)
    assert p.gang_size > 0 and p.workspace_bytes <= kdt.NOALLOC_MAX_WORKSPACE
    o1, l1 = kdt.verify_attn_noalloc(g.q_lat, g.q_pe, g.c_kv, g.k_pe, g.prefix_lens, None, cfg.softmax_scale,
                                     max_prefix_len=g.max_prefix_len, parents=g.parents, total_prefix_len=hint,
                                     schedule=2)
    o2, l2 = _run(g, total_prefix_len=hint, schedule=2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("B,H,q,lens", [(1, 1, 128, [300]),          # one row tile, the widest tree
                                        (3, 3, 100, [0, 40, 700]),    # a ragged row tile, an empty prefix
                                        (2, 16, 65, [4096, 1]),
                                        (5, 8, 9, [31, 32, 33, 64, 65])])   # lengths around the key tile
@pytest.mark.parametrize("layout", [1, 2])
def test_odd_shapes(B, H, q, lens, layout):
    cfg = synth.Config("balanced_odd", 76, "bf16", B=B, H=H, R=512, P=64, q_len=q,
                       prefix=("fixed", max(lens)), tree="uniform")
    inp = synth.generate(cfg)
    inp.prefix_lens[:] = np.asarray(lens, np.int32)
    g = GpuInputs(inp)
    for gang in (0, 1):
        o, l = _run(g, total_prefix_len=int(sum(lens)), layout=layout, schedule=2, gang_size=gang)
        _check_full(inp, o, l, f"B={B} H={H} q={q} lens={lens} layout {layout} gang {gang}")
