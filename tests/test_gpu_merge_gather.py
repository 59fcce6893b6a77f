"""GPU split stage + merge vs the oracle's merge, and the accepted-path gather
(bit-exact)."""
import numpy as np
import pytest
import torch

import oracle
from tree_verify_mla_kdt_amd import kdt, synth
from gpu_util import GpuInputs, check_close, dev, require_gpu, to_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("part_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("S", [5, 37])
def test_merge_matches_oracle_with_empty_splits(out_dtype, part_dtype, S):
    require_gpu()
    rng = synth.rng_for(5 + S)
    B, q, H, R = 3, 9, 4, 512
    M = q * H
    po = rng.standard_normal((B, S, M, R)).astype(np.float32)
    if part_dtype == torch.bfloat16:        # the partials the merge reads are exactly these values
        po = torch.from_numpy(po).to(torch.bfloat16).float().numpy()
    pl = (rng.standard_normal((B, S, M)) * 4).astype(np.float32)
    pl[rng.random((B, S, M)) < 0.3] = -np.inf
    pl[0, :, 3] = -np.inf                      # a row with no finite split
    po[pl == -np.inf] = np.nan                 # never read
    po_tiled = kdt.tile_partials(torch.from_numpy(po).to(part_dtype).to(dev()))
    assert np.array_equal(kdt.untile_partials(po_tiled, M).float().cpu().numpy(), po, equal_nan=True)
    out, lse = kdt.merge_partials(po_tiled, torch.from_numpy(pl).to(dev()), q, H, out_dtype)
    torch.cuda.synchronize()
    ro, rl = oracle.merge_partials(np.moveaxis(np.nan_to_num(po, nan=0.0), 1, 0).astype(np.float64),
                                   np.moveaxis(pl, 1, 0).astype(np.float64))
    got_o = to_f64(out).reshape(B, M, R)
    got_l = lse.cpu().numpy().reshape(B, M).astype(np.float64)
    assert np.all(got_o[0, 3] == 0) and np.isneginf(got_l[0, 3])
    fin = np.isfinite(rl)
    tol = 1e-5 if out_dtype == torch.float32 else 2e-2
    assert np.max(np.abs(got_o[fin] - ro[fin])) < tol
    assert np.max(np.abs(got_l[fin] - rl[fin])) < 1e-5


@pytest.mark.parametrize("layout", [0, 4])
@pytest.mark.parametrize("partials_f32", [False, True])
def test_partials_merge_to_full_result(partials_f32, layout):
    cfg = synth.Config("merge_cfg", 12, "bf16", B=2, H=16, R=512, P=64, q_len=17, prefix=("uniform", 100, 900),
                       tree="uniform")
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    vis, _ = kdt.build_visibility(g.parents)
    part_o, part_lse, plan = kdt.verify_partials(g.q_lat, g.q_pe, g.c_kv, g.k_pe, g.prefix_lens, vis,
                                                 cfg.softmax_scale, max_prefix_len=g.max_prefix_len,
                                                 split_keys=128, partials_f32=partials_f32, layout=layout)
    torch.cuda.synchronize()
    assert part_o.dtype == (torch.float32 if partials_f32 else torch.bfloat16)
    # each split's partial equals the oracle on that chunk of keys
    vis_np, _ = oracle.build_visibility(inp.parents)
    cache = inp.f64("cache")
    ql, qp = inp.f64("q_lat"), inp.f64("q_pe")
    po = kdt.untile_partials(part_o, cfg.q_len * cfg.H).float().cpu().numpy()
    pl = part_lse.cpu().numpy()
    for b in range(cfg.B):
        L = int(inp.prefix_lens[b])
        N = L + cfg.q_len
        ns = -(-N // plan.split_keys)
        for (t, h) in [(0, 0), (16, 15), (7, 3)]:
            m = t * cfg.H + h
            mask = oracle.key_mask(L, vis_np[b, t], cfg.q_len)
            for k in range(ns):
                a0, a1 = k * plan.split_keys, min(N, (k + 1) * plan.split_keys)
                ro, rl = oracle.attend_chunk(ql[b, t, h], qp[b, t, h], cache[b, a0:a1, :512], cache[b, a0:a1, 512:],
                                             mask[a0:a1], cfg.softmax_scale)
                if np.isneginf(rl):
                    assert np.isneginf(pl[b, k, m])
                else:
                    assert abs(pl[b, k, m] - rl) < 2e-2 and np.max(np.abs(po[b, k, m] - ro)) < 2e-2
    out, lse = kdt.merge_partials(part_o, part_lse, cfg.q_len, cfg.H, torch.bfloat16, prefix_lens=g.prefix_lens,
                                  split_keys=plan.split_keys)
    torch.cuda.synchronize()
    o_full, l_full = kdt.verify_attn(g.q_lat, g.q_pe, g.c_kv, g.k_pe, g.prefix_lens, vis, cfg.softmax_scale,
                                     max_prefix_len=g.max_prefix_len, split_keys=128, partials_f32=partials_f32,
                                     layout=layout)
    torch.cuda.synchronize()
    assert torch.equal(out, o_full) and torch.equal(lse, l_full)


# ---------------------------------------------------------------- gather

def _gather_gpu(cache_np, dtype, prefix_lens, acc, nacc, q, layers=1, seq_status=False):
    require_gpu()
    c = torch.from_numpy(cache_np.view(np.int16) if dtype == "bf16" else cache_np).to(dev())
    if dtype == "bf16":
        c = c.view(torch.bfloat16)
    pl = torch.from_numpy(np.asarray(prefix_lens, np.int32)).to(dev())
    a = torch.from_numpy(np.ascontiguousarray(acc, np.int32)).to(dev())
    n = torch.from_numpy(np.asarray(nacc, np.int32)).to(dev())
    npl = torch.full_like(pl, -1)
    st = torch.zeros_like(pl)
    if layers == 1:
        kdt.gather_accepted(c, pl, a, n, q, new_prefix_lens=npl, seq_status=st)
    else:
        kdt.gather_accepted(c[0], pl, a, n, q, num_layers=layers, layer_stride=c.stride(0),
                            new_prefix_lens=npl, seq_status=st)
    torch.cuda.synchronize()
    out = c.cpu()
    out = out.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else out.numpy()
    return out, npl.cpu().numpy(), st.cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gather_bit_exact(dtype):
    cfg = synth.config_variant(synth.CONFIGS["ragged_deep"], dtype=dtype, prefix=("uniform", 10, 300))
    inp = synth.generate(cfg)
    new, npl, st = _gather_gpu(inp.cache.copy(), dtype, inp.prefix_lens, inp.accepted, inp.n_accepted, cfg.q_len)
    ref = oracle.gather_accepted(inp.cache, inp.prefix_lens, inp.accepted, inp.n_accepted)
    assert np.array_equal(new, ref)
    assert np.array_equal(npl, inp.prefix_lens + inp.n_accepted)
    assert np.all(st == 0)


def test_gather_rotation_multilayer_and_odd_rows():
    rng = synth.rng_for(17)
    layers, B, S, C = 3, 2, 64, 37          # odd row length: 2-byte vectors
    cache = synth.f32_to_bf16_bits(rng.standard_normal((layers, B, S, C)).astype(np.float32))
    acc = np.array([[2, 0, 1, 0], [0, 3, 5, 6]], np.int32)
    nacc = [3, 4]
    pl = [10, 20]
    new, npl, _ = _gather_gpu(cache.copy(), "bf16", pl, acc, nacc, 9, layers=layers)
    for l in range(layers):
        ref = oracle.gather_accepted(cache[l], pl, acc, nacc)
        assert np.array_equal(new[l], ref)
    assert npl.tolist() == [13, 24]


def test_gather_bad_indices_flagged_and_skipped():
    rng = synth.rng_for(19)
    B, S, C = 3, 64, 576
    cache = synth.f32_to_bf16_bits(rng.standard_normal((B, S, C)).astype(np.float32))
    q = 9
    acc = np.array([[0, 12, 3], [0, 1, 2], [0, 1, 2]], np.int32)   # seq 0: index 12 >= q
    nacc = [3, 5, 2]                                                 # seq 1: n_accepted > max_acc
    pl = [5, 6, 60]                                                  # seq 2: 60 + 9 > 64 rows
    new, npl, st = _gather_gpu(cache.copy(), "bf16", pl, acc, nacc, q)
    assert st.tolist() == [kdt.KDT_SEQ_BAD_INDEX, kdt.KDT_SEQ_BAD_INDEX, kdt.KDT_SEQ_BAD_LEN]
    # seq 0: rows 0 and 2 copied, row 1 untouched
    assert np.array_equal(new[0, 5], cache[0, 5]) and np.array_equal(new[0, 6], cache[0, 6])
    assert np.array_equal(new[0, 7], cache[0, 8])
    # seq 1: clamped to 3 rows
    assert np.array_equal(new[1], oracle.gather_accepted(cache[1:2], [6], acc[1:2], [3])[0])
    # seq 2: untouched
    assert np.array_equal(new[2], cache[2])
