"""Test helpers: move generated inputs to the GPU, run the oracle on the same
bits, and compare under the stated tolerances.

Tolerances (max-abs on out and lse; relative L2 on out):
  fp32 inputs: 1e-5 max-abs.
  bf16 inputs: 2e-2 max-abs and 5e-3 relative L2.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tree_verify_mla_kdt_amd import synth

TOL_F32_ABS = 1e-5
TOL_BF16_ABS = 2e-2
TOL_BF16_REL_L2 = 5e-3


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")


def dev():
    return torch.device("cuda:0")


def tensor_of(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Exact device tensor of generated data (bf16 bit patterns or float32)."""
    if dtype == "bf16":
        return torch.from_numpy(arr.view(np.int16).copy()).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class GpuInputs:
    def __init__(self, inp: synth.Inputs, device=None):
        device = device or dev()
        cfg = inp.cfg
        self.inp = inp
        self.cfg = cfg
        self.parents = torch.from_numpy(inp.parents).to(device)
        self.prefix_lens = torch.from_numpy(inp.prefix_lens).to(device)
        self.q_lat = tensor_of(inp.q_lat, cfg.dtype, device)
        self.q_pe = tensor_of(inp.q_pe, cfg.dtype, device)
        self.cache = tensor_of(inp.cache, cfg.dtype, device)
        self.c_kv = self.cache[..., :cfg.R]
        self.k_pe = self.cache[..., cfg.R:]
        self.accepted = torch.from_numpy(inp.accepted).to(device)
        self.n_accepted = torch.from_numpy(inp.n_accepted).to(device)
        self.max_prefix_len = int(inp.prefix_lens.max())


def oracle_full(inp: synth.Inputs, vis=None):
    if vis is None:
        vis, _ = oracle.build_visibility(inp.parents)
    cache = inp.f64("cache")
    R = inp.cfg.R
    return oracle.verify_attn(inp.f64("q_lat"), inp.f64("q_pe"), cache[..., :R], cache[..., R:],
                              inp.prefix_lens, vis, inp.cfg.softmax_scale)


def oracle_by_seq(inp: synth.Inputs, vis=None):
    """The full oracle output, computed one sequence at a time (the float64
    copy of one sequence's cache at a time keeps host memory small)."""
    if vis is None:
        vis, _ = oracle.build_visibility(inp.parents)
    cfg = inp.cfg
    R = cfg.R
    q_lat, q_pe = inp.f64("q_lat"), inp.f64("q_pe")
    o = np.zeros(q_lat.shape, np.float64)
    lse = np.zeros(q_lat.shape[:3], np.float64)
    for b in range(cfg.B):
        cb = synth.to_f64(inp.cache[b], cfg.dtype)
        o[b:b + 1], lse[b:b + 1] = oracle.verify_attn(q_lat[b:b + 1], q_pe[b:b + 1], cb[None, :, :R], cb[None, :, R:],
                                                      inp.prefix_lens[b:b + 1], vis[b:b + 1], cfg.softmax_scale)
    return o, lse


def oracle_rows(inp: synth.Inputs, rows, vis=None):
    if vis is None:
        vis, _ = oracle.build_visibility(inp.parents)
    cfg = inp.cfg
    R = cfg.R
    cache = inp.cache
    # convert lazily per sequence to keep memory small
    q_lat, q_pe = inp.f64("q_lat"), inp.f64("q_pe")
    res = {}
    for b in sorted({r[0] for r in rows}):
        cb = synth.to_f64(cache[b], cfg.dtype)          # one sequence at a time keeps memory small
        mine = [r for r in rows if r[0] == b]
        o, l = oracle.verify_attn_rows(q_lat[b:b + 1], q_pe[b:b + 1], cb[None, :, :R], cb[None, :, R:],
                                       inp.prefix_lens[b:b + 1], vis[b:b + 1], cfg.softmax_scale,
                                       [(0, t, h) for (_, t, h) in mine])
        for k, r in enumerate(mine):
            res[r] = (o[k], l[k])
    return np.stack([res[r][0] for r in rows]), np.asarray([res[r][1] for r in rows])


def check_close(dtype: str, got_o, ref_o, got_lse, ref_lse, what=""):
    got_o = np.asarray(got_o, dtype=np.float64)
    ref_o = np.asarray(ref_o, dtype=np.float64)
    err = np.max(np.abs(got_o - ref_o)) if got_o.size else 0.0
    lerr = np.max(np.abs(np.asarray(got_lse, np.float64) - np.asarray(ref_lse, np.float64))) if np.size(ref_lse) else 0.0
    assert np.all(np.isfinite(got_o)), f"{what}: non-finite output"
    if dtype == "f32":
        assert err <= TOL_F32_ABS, f"{what}: out max-abs {err:.3e} > {TOL_F32_ABS}"
        assert lerr <= TOL_F32_ABS, f"{what}: lse max-abs {lerr:.3e} > {TOL_F32_ABS}"
        return err, lerr, 0.0
    rel = np.linalg.norm(got_o - ref_o) / max(np.linalg.norm(ref_o), 1e-30)
    assert err <= TOL_BF16_ABS, f"{what}: out max-abs {err:.3e} > {TOL_BF16_ABS}"
    assert rel <= TOL_BF16_REL_L2, f"{what}: out rel-L2 {rel:.3e} > {TOL_BF16_REL_L2}"
    assert lerr <= TOL_BF16_ABS, f"{what}: lse max-abs {lerr:.3e} > {TOL_BF16_ABS}"
    return err, lerr, rel


def sample_rows(inp: synth.Inputs, n: int, seed: int = 0):
    """Sampled (b, t, h) rows covering first/last tokens, heads and sequences."""
    cfg = inp.cfg
    rng = synth.rng_for(900 + seed)
    rows = {(0, 0, 0), (cfg.B - 1, cfg.q_len - 1, cfg.H - 1), (0, cfg.q_len - 1, 0), (cfg.B - 1, 0, cfg.H - 1)}
    while len(rows) < n:
        rows.add((int(rng.integers(cfg.B)), int(rng.integers(cfg.q_len)), int(rng.integers(cfg.H))))
    return sorted(rows)
