"""GPU: kdt_verify_attn_noalloc (the library's fixed device workspace instead
of a caller's) against kdt_verify_attn on the same inputs, through the C ABI:
two calls in a row, the second smaller, both bit-identical to the existing
entry point; an oversized plan and the in-kernel merge are refused."""
import numpy as np
import pytest
import torch

from tree_verify_mla_kdt_amd import kdt, synth
from gpu_util import GpuInputs, require_gpu

pytestmark = pytest.mark.gpu


def _both(g, **kw):
    args = (g.q_lat, g.q_pe, g.c_kv, g.k_pe, g.prefix_lens, None, g.cfg.softmax_scale)
    o1, l1 = kdt.verify_attn(*args, max_prefix_len=g.max_prefix_len, parents=g.parents, **kw)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    kdt.verify_attn_noalloc(*args, max_prefix_len=g.max_prefix_len, parents=g.parents, out=o2, lse=l2, **kw)
    torch.cuda.synchronize()
    return o1, l1, o2, l2


def test_noalloc_matches_verify_attn_two_calls():
    require_gpu()
    big = GpuInputs(synth.generate(synth.CONFIGS["max_budget"]))
    small_cfg = synth.Config("noalloc_small", 41, "bf16", B=2, H=16, R=512, P=64, q_len=17,
                             prefix=("uniform", 150, 700), tree="uniform")
    small = GpuInputs(synth.generate(small_cfg))
    for g, kw in ((big, {}), (small, {"split_keys": 64})):
        d, _, _ = kdt._verify_prepare(g.q_lat, g.q_pe, g.c_kv, g.k_pe, g.prefix_lens, None, g.cfg.softmax_scale,
                                      g.max_prefix_len, None, None, None, kw.get("split_keys", 0), parents=g.parents)
        p = kdt.verify_plan(d)
        assert p.direct == 0 and 0 < p.workspace_bytes <= kdt.NOALLOC_MAX_WORKSPACE
        o1, l1, o2, l2 = _both(g, **kw)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), g.cfg.name
        assert torch.isfinite(o2).all()


def test_noalloc_refuses_oversized_plan_and_inkernel_merge():
    require_gpu()
    g = GpuInputs(synth.generate(synth.CONFIGS["max_budget"]))
    args = (g.q_lat, g.q_pe, g.c_kv, g.k_pe, g.prefix_lens, None, g.cfg.softmax_scale)
    with pytest.raises(kdt.KdtError) as e:                  # 131 splits of partials: far beyond the fixed array
        kdt.verify_attn_noalloc(*args, max_prefix_len=g.max_prefix_len, parents=g.parents, split_keys=32)
    assert e.value.code == 3
    d, out, lse = kdt._verify_prepare(*args, g.max_prefix_len, None, None, None, 0, parents=g.parents,
                                      merge_mode=1)
    import ctypes
    assert kdt.lib().kdt_verify_attn_noalloc(ctypes.byref(d), kdt._stream(None)) == 2
