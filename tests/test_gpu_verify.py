"""GPU tree-verify attention vs the float64 oracle.

Full element-by-element comparisons at sizes the oracle finishes in seconds
(several key tiles, ragged tails, several row tiles), every configuration at
its full size (every row; the largest ones run the oracle one sequence at a
time), the AR (q_len = 1) case, forced split counts, and the invariants: masked keys get
exactly zero weight (bit-identical output), chain == successive AR calls,
prefix permutation, gather-then-AR == tree row.
"""
import numpy as np
import pytest
import torch

import oracle
from tree_verify_mla_kdt_amd import kdt, synth
from gpu_util import (GpuInputs, check_close, oracle_by_seq, oracle_full, oracle_rows, require_gpu, sample_rows,
                      to_f64)

pytestmark = pytest.mark.gpu


def run_gpu(g: GpuInputs, split_keys=0, vis=None, max_prefix_len=None, seq_status=None, layout=0,
            partials_f32=False, from_parents=False):
    """from_parents: hand the verify the parent pointers (the split kernel
    derives the masks, as in the bench step) instead of kdt_build_visibility's
    masks."""
    require_gpu()
    if vis is None and not from_parents:
        vis, _ = kdt.build_visibility(g.parents)
    out, lse = kdt.verify_attn(g.q_lat, g.q_pe, g.c_kv, g.k_pe, g.prefix_lens, vis, g.cfg.softmax_scale,
                               max_prefix_len=g.max_prefix_len if max_prefix_len is None else max_prefix_len,
                               split_keys=split_keys, seq_status=seq_status, layout=layout,
                               partials_f32=partials_f32, parents=g.parents if from_parents else None)
    torch.cuda.synchronize()
    return to_f64(out), lse.cpu().numpy().astype(np.float64)


def small_cfg(dtype="bf16", B=2, H=16, R=512, P=64, q=17, prefix=("fixed", 200), tree="uniform", index=11):
    return synth.Config(f"small_{dtype}_{R}_{q}", index, dtype, B=B, H=H, R=R, P=P, q_len=q, prefix=prefix,
                        tree=tree)


# ---------------------------------------------------------------- full parity, small sizes

@pytest.mark.parametrize("split_keys", [0, 64])
def test_tiny_fp32_config(split_keys):
    inp = synth.generate(synth.CONFIGS["tiny_fp32"])
    g = GpuInputs(inp)
    o, l = run_gpu(g, split_keys=split_keys)
    ro, rl = oracle_full(inp)
    check_close("f32", o, ro, l, rl, "tiny_fp32")


@pytest.mark.parametrize("q,tree", [(1, "chain"), (9, "uniform"), (17, "star"), (33, "deep_chain"),
                                    (65, "best_first"), (65, "chain"), (100, "uniform"), (128, "uniform")])
def test_bf16_full_parity_tree_shapes(q, tree):
    cfg = small_cfg(q=q, tree=tree, prefix=("uniform", 0, 300), B=3, H=8, index=20 + q)
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    o, l = run_gpu(g)
    ro, rl = oracle_full(inp)
    check_close("bf16", o, ro, l, rl, f"q={q} {tree}")


@pytest.mark.parametrize("partials_f32", [False, True])
@pytest.mark.parametrize("split_keys", [0, 32, 64, 96, 128, 192, 288, 1024])
def test_bf16_split_counts_agree(split_keys, partials_f32):
    cfg = small_cfg(q=33, tree="deep_chain", prefix=("uniform", 40, 700), B=3, H=16, index=31)
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    o, l = run_gpu(g, split_keys=split_keys, partials_f32=partials_f32)
    ro, rl = oracle_full(inp)
    check_close("bf16", o, ro, l, rl, f"split_keys={split_keys} partials_f32={partials_f32}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_rank_shapes(dtype):
    cfg = small_cfg(dtype=dtype, R=64, P=16, H=4, q=9, prefix=("uniform", 0, 130), B=4, index=41)
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    for sk in (0, 64):
        o, l = run_gpu(g, split_keys=sk)
        ro, rl = oracle_full(inp)
        check_close(dtype, o, ro, l, rl, f"{dtype} R=64 split={sk}")


def test_heads_not_multiple_of_tile_and_empty_prefix():
    # M = q*H = 7*3 = 21 rows: one partial row tile; prefix 0 for one sequence
    cfg = small_cfg(q=7, H=3, prefix=("fixed", 0), B=2, index=51)
    inp = synth.generate(cfg, prefix_override=[0, 77])
    g = GpuInputs(inp)
    o, l = run_gpu(g)
    ro, rl = oracle_full(inp)
    check_close("bf16", o, ro, l, rl, "H=3 q=7")


def test_strided_fused_and_separate_caches():
    cfg = small_cfg(q=17, H=16, prefix=("fixed", 333), B=2, index=61)
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    o1, l1 = run_gpu(g)
    # separate contiguous c_kv / k_pe buffers must give bit-identical results
    g.c_kv = g.cache[..., :cfg.R].contiguous()
    g.k_pe = g.cache[..., cfg.R:].contiguous()
    o2, l2 = run_gpu(g)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("layout", [1, 2, 3, 4])
def test_query_layouts_give_identical_results(layout):
    """Queries with padded rows (one uniform row stride larger than R) and in a
    head-major buffer (token stride smaller than the head stride) give the
    same bits as contiguous queries: the 64-row layout copies uniformly
    strided query rows through LDS and loads the others directly."""
    cfg = small_cfg(q=9, H=16, prefix=("uniform", 40, 400), B=3, index=62)
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    o1, l1 = run_gpu(g, layout=layout)
    B, q, H, R, P = cfg.B, cfg.q_len, cfg.H, cfg.R, cfg.P
    # padded rows: [B, q, H, R + 32] and [B, q, H, P + 16] buffers
    ql_pad = torch.zeros((B, q, H, R + 32), dtype=g.q_lat.dtype, device=g.q_lat.device)
    qp_pad = torch.zeros((B, q, H, P + 16), dtype=g.q_pe.dtype, device=g.q_pe.device)
    ql_pad[..., :R] = g.q_lat
    qp_pad[..., :P] = g.q_pe
    q_lat0, q_pe0 = g.q_lat, g.q_pe
    g.q_lat, g.q_pe = ql_pad[..., :R], qp_pad[..., :P]
    o2, l2 = run_gpu(g, layout=layout)
    # head-major buffers viewed as [B, q, H, *]
    g.q_lat = q_lat0.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    g.q_pe = q_pe0.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    o3, l3 = run_gpu(g, layout=layout)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)
    ro, rl = oracle_full(inp)
    check_close("bf16", o1, ro, l1, rl, f"layout {layout}")


def _growing_scores_inputs(q, H, L, B=2, index=63):
    """Scores that rise by far more than 2^32 in weight after the first key
    tiles: q_lat is all ones, c_kv rows are a per-key level plus small noise,
    with level 0 for the first keys and 3 from key L // 3 on, so the reference
    a split takes from its first tile is exceeded later and the split is
    redone against the exact maximum."""
    cfg = small_cfg(q=q, H=H, prefix=("fixed", L), B=B, index=index)
    inp = synth.generate(cfg)
    rng = synth.rng_for(63)
    R, P = cfg.R, cfg.P
    S = inp.cache.shape[1]
    level = np.where(np.arange(S) < L // 3, 0.0, 3.0).astype(np.float32)
    c = level[None, :, None] + 0.02 * rng.standard_normal((B, S, R + P)).astype(np.float32)
    c[..., R:] = 0.0
    inp.cache = synth.f32_to_bf16_bits(c)
    inp.q_lat = synth.f32_to_bf16_bits(np.ones(inp.q_lat.shape, np.float32))
    inp.q_pe = synth.f32_to_bf16_bits(np.zeros(inp.q_pe.shape, np.float32))
    return inp


@pytest.mark.parametrize("layout,split_keys", [(1, 0), (2, 0), (3, 0), (4, 0), (1, 256), (2, 256), (3, 256), (4, 256),
                                               (2, 64), (3, 64), (4, 64), (1, 32), (2, 96), (4, 32), (4, 96)])
def test_redo_when_scores_outgrow_the_reference(layout, split_keys):
    inp = _growing_scores_inputs(q=9, H=16, L=900)
    g = GpuInputs(inp)
    ro, rl = oracle_full(inp)
    # the weight sits on the level-3 keys: every output is near 3 (the largest
    # outputs of the suite, so the bf16 partials' rounding is largest here)
    assert np.all(np.abs(ro - 3.0) < 0.1)
    for pf in (False, True):
        o, l = run_gpu(g, split_keys=split_keys, layout=layout, partials_f32=pf)
        check_close("bf16", o, ro, l, rl, f"layout {layout} split {split_keys} partials_f32={pf}")


# ---------------------------------------------------------------- full-size configurations
#
# Each runs both routes to the masks: kdt_build_visibility's, and the split
# kernel deriving them from the parents (the bench step's launch
# configuration); the two must agree bit for bit.

def _both_routes(g, **kw):
    o, l = run_gpu(g, **kw)
    o2, l2 = run_gpu(g, from_parents=True, **kw)
    assert np.array_equal(o, o2) and np.array_equal(l, l2), "mask routes disagree"
    return o, l


def test_config_max_budget_full():
    inp = synth.generate(synth.CONFIGS["max_budget"])
    g = GpuInputs(inp)
    o, l = _both_routes(g)
    ro, rl = oracle_full(inp)
    check_close("bf16", o, ro, l, rl, "max_budget")


def test_config_batched_full():
    inp = synth.generate(synth.CONFIGS["batched"])
    g = GpuInputs(inp)
    o, l = _both_routes(g)
    ro, rl = oracle_full(inp)
    check_close("bf16", o, ro, l, rl, "batched")


@pytest.mark.parametrize("name", ["long_ctx", "ragged_deep"])
def test_config_large_full(name):
    """Every row of the two largest configurations against the float64 oracle
    (run one sequence at a time: a few seconds of host time)."""
    inp = synth.generate(synth.CONFIGS[name])
    g = GpuInputs(inp)
    o, l = _both_routes(g)
    ro, rl = oracle_by_seq(inp)
    check_close("bf16", o, ro, l, rl, name)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))


@pytest.mark.parametrize("name", ["max_budget", "long_ctx"])
def test_ar_degenerate_q1(name):
    cfg = synth.config_variant(synth.CONFIGS[name], q_len=1)
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    o, l = _both_routes(g)
    ro, rl = oracle_by_seq(inp)
    check_close("bf16", o, ro, l, rl, f"{name} q=1")


# ---------------------------------------------------------------- invariants

def test_masked_keys_have_exactly_zero_weight():
    cfg = small_cfg(q=33, tree="star", prefix=("fixed", 150), B=2, H=16, index=71)
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    o1, l1 = run_gpu(g, split_keys=64)
    L, q = int(inp.prefix_lens[0]), cfg.q_len
    # rows past the tree: invisible to every token
    g.cache[:, L + q:] = 300.0
    o2, l2 = run_gpu(g, split_keys=64)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # in a star, node j >= 1 is seen only by token j
    j = 5
    g.cache[:, L + j] = -250.0
    o3, l3 = run_gpu(g, split_keys=64)
    others = [t for t in range(q) if t != j]
    assert np.array_equal(o3[:, others], o1[:, others]) and np.array_equal(l3[:, others], l1[:, others])
    assert not np.array_equal(o3[:, j], o1[:, j])


def test_chain_equals_successive_ar_calls():
    cfg = small_cfg(q=9, tree="chain", prefix=("fixed", 260), B=1, H=16, index=81)
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    o, l = run_gpu(g)
    one = torch.ones((1, 1, 1), dtype=torch.int64, device=g.q_lat.device)
    for t in range(cfg.q_len):
        out, lse = kdt.verify_attn(g.q_lat[:, t:t + 1], g.q_pe[:, t:t + 1], g.c_kv, g.k_pe,
                                   g.prefix_lens + t, one, cfg.softmax_scale, max_prefix_len=260 + t)
        torch.cuda.synchronize()
        check_close("bf16", to_f64(out)[0, 0], o[0, t], lse.cpu().numpy()[0, 0], l[0, t], f"AR step {t}")


def test_prefix_permutation_invariance():
    cfg = small_cfg(q=17, prefix=("fixed", 500), B=1, H=16, index=91)
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    o1, l1 = run_gpu(g)
    perm = torch.from_numpy(synth.rng_for(3).permutation(500)).to(g.cache.device)
    g.cache[:, :500] = g.cache[:, perm]
    o2, l2 = run_gpu(g)
    check_close("bf16", o2, o1, l2, l1, "prefix permutation")


def test_gather_then_ar_equals_tree_row():
    cfg = small_cfg(q=17, tree="uniform", prefix=("fixed", 123), B=1, H=16, index=95)
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    o, l = run_gpu(g)
    _, depth = oracle.build_visibility(inp.parents)
    one = torch.ones((1, 1, 1), dtype=torch.int64, device=g.q_lat.device)
    for t in (0, 5, 16):
        g2 = GpuInputs(inp)
        path = synth.path_to(inp.parents[0], t)
        acc = torch.zeros((1, cfg.q_len), dtype=torch.int32, device=g2.cache.device)
        acc[0, :len(path)] = torch.from_numpy(path)
        n = torch.tensor([len(path)], dtype=torch.int32, device=g2.cache.device)
        kdt.gather_accepted(g2.cache, g2.prefix_lens, acc, n, cfg.q_len)
        d = int(depth[0, t])
        out, lse = kdt.verify_attn(g2.q_lat[:, t:t + 1], g2.q_pe[:, t:t + 1], g2.c_kv, g2.k_pe,
                                   g2.prefix_lens + d, one, cfg.softmax_scale, max_prefix_len=123 + d)
        torch.cuda.synchronize()
        check_close("bf16", to_f64(out)[0, 0], o[0, t], lse.cpu().numpy()[0, 0], l[0, t], f"path to {t}")


def test_bad_prefix_lengths_are_skipped_and_flagged():
    cfg = small_cfg(q=9, prefix=("fixed", 100), B=3, H=4, index=97)
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    st = torch.zeros(3, dtype=torch.int32, device=g.q_lat.device)
    g.prefix_lens[1] = 150          # beyond the max_prefix_len bound passed below
    g.prefix_lens[2] = -3
    for sk in (0, 64):
        st.zero_()
        o, l = run_gpu(g, split_keys=sk, max_prefix_len=100, seq_status=st)
        assert st.cpu().tolist() == [0, kdt.KDT_SEQ_BAD_LEN, kdt.KDT_SEQ_BAD_LEN]
        assert np.all(o[1:] == 0) and np.all(np.isneginf(l[1:]))
        ro, rl = oracle_full(synth.Inputs(cfg, inp.parents[:1], inp.prefix_lens[:1], inp.q_lat[:1],
                                          inp.q_pe[:1], inp.cache[:1], inp.accepted[:1], inp.n_accepted[:1]))
        check_close("bf16", o[:1], ro, l[:1], rl, f"good sequence, split={sk}")


@pytest.mark.parametrize("q,H", [(3, 16), (4, 16), (65, 1)])
@pytest.mark.parametrize("split_keys", [0, 32, 64, 4096])
def test_short_row_counts_all_split_modes(q, H, split_keys):
    # q*H = 48 (second 32-row block half filled), 64 (exactly two blocks: the
    # column-split layout of a workgroup) and 65 (just past it, the full
    # layout); forced small splits, automatic, and one split (direct output)
    cfg = small_cfg(q=q, H=H, tree="uniform", prefix=("uniform", 100, 700), B=3, index=101 + q + H)
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    o, l = run_gpu(g, split_keys=split_keys)
    ro, rl = oracle_full(inp)
    check_close("bf16", o, ro, l, rl, f"q={q} H={H} split_keys={split_keys}")


@pytest.mark.parametrize("layout", [1, 2, 3, 4])
@pytest.mark.parametrize("q,H,tree", [(1, 16, "chain"), (17, 16, "uniform"), (65, 16, "best_first"),
                                      (33, 3, "deep_chain")])
def test_forced_layouts_match_oracle(layout, q, H, tree):
    cfg = small_cfg(q=q, H=H, tree=tree, prefix=("uniform", 50, 900), B=2, index=140 + q + H)
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    ro, rl = oracle_full(inp)
    for sk in (0, 128):
        o, l = run_gpu(g, split_keys=sk, layout=layout)
        check_close("bf16", o, ro, l, rl, f"layout={layout} q={q} H={H} split_keys={sk}")


def test_config_max_budget_all_layouts_agree():
    inp = synth.generate(synth.CONFIGS["max_budget"])
    g = GpuInputs(inp)
    ro, rl = oracle_full(inp)
    for layout in (1, 2, 3, 4):
        o, l = run_gpu(g, layout=layout)
        check_close("bf16", o, ro, l, rl, f"max_budget layout {layout}")


# ---------------------------------------------------------------- masks derived from parents

@pytest.mark.parametrize("layout", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("q,H,tree,split_keys", [(1, 16, "chain", 0), (17, 16, "uniform", 0),
                                                 (65, 16, "best_first", 64), (100, 4, "uniform", 0),
                                                 (128, 2, "deep_chain", 128), (33, 3, "deep_chain", 0)])
def test_masks_from_parents_match_given_masks(layout, q, H, tree, split_keys):
    """vis = None with parents: the split kernel derives the masks itself and
    the result is bit-identical to the one with kdt_build_visibility's masks
    (only splits that reach the tree derive them)."""
    cfg = small_cfg(q=q, H=H, tree=tree, prefix=("uniform", 30, 700), B=3, index=300 + q + H)
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    vis, _ = kdt.build_visibility(g.parents)
    args = (g.q_lat, g.q_pe, g.c_kv, g.k_pe, g.prefix_lens)
    o1, l1 = kdt.verify_attn(*args, vis, cfg.softmax_scale, max_prefix_len=g.max_prefix_len,
                             split_keys=split_keys, layout=layout)
    st = torch.zeros(cfg.B, dtype=torch.int32, device=g.parents.device)
    o2, l2 = kdt.verify_attn(*args, None, cfg.softmax_scale, max_prefix_len=g.max_prefix_len,
                             split_keys=split_keys, layout=layout, parents=g.parents, seq_status=st)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert st.cpu().tolist() == [0] * cfg.B
    ro, rl = oracle_full(inp)
    check_close("bf16", to_f64(o2), ro, l2.cpu().numpy().astype(np.float64), rl, f"parents layout={layout} q={q}")


def test_bad_trees_from_parents_are_flagged_like_the_mask_kernel():
    cfg = small_cfg(q=9, H=4, tree="uniform", prefix=("fixed", 100), B=4, index=77)
    inp = synth.generate(cfg)
    par = inp.parents.copy()
    par[1, 0] = 3                      # root with a parent
    par[2, 4], par[2, 6] = 6, 4        # a cycle through forward parents
    par[3, 2] = -7                     # out of range
    g = GpuInputs(inp)
    g.parents = torch.from_numpy(par).to(g.parents.device)
    st1 = torch.zeros(cfg.B, dtype=torch.int32, device=g.parents.device)
    vis, _ = kdt.build_visibility(g.parents, seq_status=st1)
    args = (g.q_lat, g.q_pe, g.c_kv, g.k_pe, g.prefix_lens)
    o1, l1 = kdt.verify_attn(*args, vis, cfg.softmax_scale, max_prefix_len=g.max_prefix_len)
    st2 = torch.zeros_like(st1)
    o2, l2 = kdt.verify_attn(*args, None, cfg.softmax_scale, max_prefix_len=g.max_prefix_len,
                             parents=g.parents, seq_status=st2)
    torch.cuda.synchronize()
    bad = kdt.KDT_SEQ_BAD_TREE
    assert st1.cpu().tolist() == [0, bad, bad, bad] and st2.cpu().tolist() == st1.cpu().tolist()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("layout", [0, 1, 2, 4])
def test_many_sequences_more_workgroups_than_units(layout):
    """257 short ragged sequences: the grid holds more workgroups than the GPU
    has compute units, so several rounds run and every index mapping (XCD
    order, row tiles, splits) is exercised past the first round."""
    cfg = small_cfg(q=5, H=8, tree="uniform", prefix=("uniform", 0, 300), B=257, index=401)
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    ro, rl = oracle_full(inp)
    for sk in (0, 64):
        o, l = run_gpu(g, split_keys=sk, layout=layout, from_parents=True)
        check_close("bf16", o, ro, l, rl, f"B=257 layout={layout} split_keys={sk}")


def test_group_order_past_32_bit_products():
    """More than 46340 (sequence, split) groups: the product behind the order
    in which workgroups visit the groups no longer fits in 32 bits and the
    kernel takes its 64-bit path; sampled rows across the batch, the last
    sequences included, must still match the oracle."""
    cfg = small_cfg(q=1, H=16, R=64, P=16, tree="chain", prefix=("uniform", 1, 512), B=2728, index=402)
    inp = synth.generate(cfg)
    inp.prefix_lens[-1] = 512                      # the longest length sets the split count
    g = GpuInputs(inp)
    d, _, _ = kdt._verify_prepare(g.q_lat, g.q_pe, g.c_kv, g.k_pe, g.prefix_lens, None, cfg.softmax_scale,
                                  g.max_prefix_len, None, None, None, 32, parents=g.parents)
    p = kdt.verify_plan(d)
    assert p.max_splits * cfg.B > 46340 and p.gang_size == 0
    o, l = run_gpu(g, split_keys=32)
    rows = sorted(set(sample_rows(inp, 96, seed=7)) | {(b, 0, h) for b in (cfg.B - 2, cfg.B - 1) for h in (0, 15)})
    ro, rl = oracle_rows(inp, rows)
    go = np.stack([o[b, t, h] for (b, t, h) in rows])
    gl = np.asarray([l[b, t, h] for (b, t, h) in rows])
    check_close("bf16", go, ro, gl, rl, "B=2728 fixed splits of 32 keys")
    assert np.isfinite(o).all() and np.isfinite(l).all()


@pytest.mark.parametrize("layout", [1, 2, 3, 4])
def test_tight_cache_capacity(layout):
    """The cache holds exactly max_b(L_b + q_len) rows, not a multiple of the
    32-key tile: the last split of the longest sequence ends at the cache's
    last row, so its copy descriptor spans only rows inside the cache and the
    start-up copies that assume two full tiles are not used there."""
    cfg = small_cfg(q=17, H=16, tree="uniform", B=3, index=431)
    inp = synth.generate(cfg, prefix_override=[699, 301, 13], cap_round=1)
    assert inp.S_cap == 699 + 17 and inp.S_cap % 32 != 0
    g = GpuInputs(inp)
    ro, rl = oracle_full(inp)
    for sk in (0, 32, 96):
        for fp in (False, True):
            o, l = run_gpu(g, split_keys=sk, layout=layout, from_parents=fp)
            check_close("bf16", o, ro, l, rl, f"tight capacity layout={layout} split_keys={sk} parents={fp}")


@pytest.mark.parametrize("layout", [0, 1, 2, 4])
def test_large_row_stride_offsets(layout):
    """Cache rows 2 MB apart (2^20 bf16 elements, only the first R + P of each
    holding data): the largest split allowed, 992 keys, then spans close to
    2^31 bytes, the limit of the kernel's 32-bit row offsets, so the largest
    offsets its copies compute are exercised.  The automatic split size and
    that largest one must both match the oracle."""
    cfg = small_cfg(q=17, H=16, tree="uniform", B=1, prefix=("fixed", 2000), index=451)
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    stride = 1 << 20
    big = torch.empty((1, g.cache.shape[1], stride), dtype=g.cache.dtype, device=g.cache.device)   # 4.3 GB
    big[..., :cfg.R + cfg.P] = g.cache
    g.c_kv = big[..., :cfg.R]
    g.k_pe = big[..., cfg.R:cfg.R + cfg.P]
    limit = (2 ** 31 - 1) // (stride * 2) // 32 * 32
    assert limit == 992
    ro, rl = oracle_full(inp)
    try:
        for sk in (0, limit):
            o, l = run_gpu(g, split_keys=sk, layout=layout)
            check_close("bf16", o, ro, l, rl, f"2 MB row stride layout={layout} split_keys={sk}")
    finally:
        del g, big
        torch.cuda.empty_cache()

