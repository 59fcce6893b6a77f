"""GPU: the cross-split merge inside the split kernel.

With merge_mode 1, and when every split workgroup of a launch fits on the
device at once, kdt_verify_attn merges the partials in the same kernel (the
split workgroups of a row tile meet at a state word in the workspace and
share the merge).  The
result must equal, bit for bit, the separate merge kernel's, also when every
workgroup gives up waiting at once (the last one out then merges everything),
and the float64 oracle within the bf16 tolerances; the counts in the state
words must be left at zero so one workspace serves any sequence of calls.
"""
import numpy as np
import pytest
import torch

from tree_verify_mla_kdt_amd import kdt, synth
from gpu_util import GpuInputs, check_close, oracle_by_seq, require_gpu, to_f64

pytestmark = pytest.mark.gpu


def _run(g, ws, **kw):
    # (the fused merge is a split-schedule option: the separate merge it is
    # compared with must see the same splits, not the balanced schedule)
    kw.setdefault("schedule", 1)
    out, lse = kdt.verify_attn(g.q_lat, g.q_pe, g.c_kv, g.k_pe, g.prefix_lens, None, g.cfg.softmax_scale,
                               max_prefix_len=g.max_prefix_len, workspace=ws, parents=g.parents, **kw)
    torch.cuda.synchronize()
    return out.clone(), lse.clone()


def _plan(g, **kw):
    kw.setdefault("schedule", 1)
    d, _, _ = kdt._verify_prepare(g.q_lat, g.q_pe, g.c_kv, g.k_pe, g.prefix_lens, None, g.cfg.softmax_scale,
                                  g.max_prefix_len, None, None, None, kw.pop("split_keys", 0), parents=g.parents,
                                  **kw)
    return kdt.verify_plan(d)


def _counters(ws, plan, B):
    """The counts of every row tile's merge state word (the generation bit,
    bit 31, alternates from call to call; the counts must be back at zero)."""
    n_rt = -(-plan.rows // (128 if plan.layout == 1 else 64))
    c = ws[plan.counter_offset:plan.counter_offset + B * n_rt * 4].view(torch.int32)
    return c.cpu().numpy() & 0x7FFFFFFF


CASES = [
    ("max_budget", {}),                                   # 11 splits x 17 row tiles
    ("max_budget:q1", {}),                                # AR: more than sixteen splits (a workgroup per item)
    ("ragged_deep", {}),                                  # ragged: each sequence its own split count
    ("long_ctx:q1", {}),
    ("max_budget", {"split_keys": 256, "layout": 1}),     # 128-row layout
    ("max_budget", {"split_keys": 320, "layout": 2}),
    ("max_budget", {"split_keys": 416, "partials_f32": True}),
]


def _inputs(name):
    base, _, var = name.partition(":")
    cfg = synth.CONFIGS[base]
    if var == "q1":
        cfg = synth.config_variant(cfg, q_len=1)
    return synth.generate(cfg)


@pytest.mark.parametrize("name,kw", CASES)
def test_fused_merge_equals_separate_merge(name, kw):
    require_gpu()
    inp = _inputs(name)
    g = GpuInputs(inp)
    p = _plan(g, merge_mode=1, **kw)
    assert p.direct == 0 and p.fused_merge == 1, "this case is meant to fuse the merge"
    assert _plan(g, **kw).fused_merge == 0                # (not the default)
    ws = torch.zeros(p.workspace_bytes, dtype=torch.uint8, device=g.q_lat.device)
    o1, l1 = _run(g, ws, merge_mode=1, **kw)
    assert np.all(_counters(ws, p, inp.cfg.B) == 0)
    o2, l2 = _run(g, ws, merge_mode=1, **kw)              # the same workspace again
    o3, l3 = _run(g, None, **kw)                          # the separate merge kernel
    o4, l4 = _run(g, ws, merge_mode=1, merge_wait_us=-1, **kw)   # nobody waits: the last arriver merges all
    assert np.all(_counters(ws, p, inp.cfg.B) == 0)
    for o, l in ((o2, l2), (o3, l3), (o4, l4)):
        assert torch.equal(o1, o), name
        assert torch.equal(l1, l), name
    if name in ("max_budget", "ragged_deep", "long_ctx:q1") and not kw:
        ro, rl = oracle_by_seq(inp)
        check_close("bf16", to_f64(o1), ro, l1.cpu().numpy().astype(np.float64), rl, name)


def test_fused_merge_bad_lengths_and_shorter_sequences():
    """A skipped sequence (bad prefix length) and sequences with fewer splits
    than the launch's maximum, in one fused launch."""
    require_gpu()
    cfg = synth.Config("fused_ragged", 31, "bf16", B=5, H=16, R=512, P=64, q_len=17,
                       prefix=("uniform", 40, 2000), tree="uniform")
    inp = synth.generate(cfg)
    g = GpuInputs(inp)
    L = inp.prefix_lens.copy()
    bad = L.copy()
    bad[2] = -5
    g.prefix_lens = torch.from_numpy(bad).to(g.q_lat.device)
    p = _plan(g, split_keys=128, layout=1, merge_mode=1)
    assert p.fused_merge == 1
    ws = torch.zeros(p.workspace_bytes, dtype=torch.uint8, device=g.q_lat.device)
    st = torch.zeros(cfg.B, dtype=torch.int32, device=g.q_lat.device)
    o1, l1 = _run(g, ws, split_keys=128, layout=1, seq_status=st, merge_mode=1)
    o2, l2 = _run(g, None, split_keys=128, layout=1)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert np.all(_counters(ws, p, cfg.B) == 0)
    s = st.cpu().numpy()
    assert s[2] == kdt.KDT_SEQ_BAD_LEN and np.all(np.delete(s, 2) == 0)
    assert torch.all(o1[2] == 0) and torch.all(torch.isneginf(l1[2]))
    ro, rl = oracle_by_seq(inp)
    keep = [b for b in range(cfg.B) if b != 2]
    check_close("bf16", to_f64(o1)[keep], ro[keep], l1.cpu().numpy().astype(np.float64)[keep], rl[keep], "fused")
