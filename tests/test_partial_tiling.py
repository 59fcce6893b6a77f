"""Host check of the tiled partial layouts (float32 and bf16) the split stage
writes and the merge reads: the binding's tile/untile helpers against the
element formulas, and their round trip."""
import numpy as np
import pytest
import torch

from tree_verify_mla_kdt_amd import kdt


def _pos_f32(r, c):
    return 256 * (c // 8) + 128 * ((c // 4) % 2) + 4 * r + c % 4


def _pos_bf16(r, c):
    return 512 * (c // 16) + 8 * (r + 32 * ((c // 4) % 2)) + 4 * ((c // 8) % 2) + c % 4


@pytest.mark.parametrize("dtype,pos", [(torch.float32, _pos_f32), (torch.bfloat16, _pos_bf16)])
@pytest.mark.parametrize("M,R", [(36, 64), (70, 512), (32, 16 * 3)])
def test_tiling_matches_formula(dtype, pos, M, R):
    B, S = 2, 3
    vals = torch.arange(B * S * M * R, dtype=torch.float64).remainder(251).to(dtype).reshape(B, S, M, R)
    tiled = kdt.tile_partials(vals)
    nblk = kdt.partial_blocks(M)
    assert tiled.shape == (B, S, nblk, 32 * R) and tiled.is_contiguous()
    t = tiled.numpy() if dtype == torch.float32 else tiled.view(torch.int16).numpy()
    v = vals.numpy() if dtype == torch.float32 else vals.view(torch.int16).numpy()
    rng = np.random.default_rng(M + R)
    for _ in range(300):
        b, s, m, c = rng.integers(B), rng.integers(S), rng.integers(M), rng.integers(R)
        assert t[b, s, m // 32, pos(m % 32, c)] == v[b, s, m, c]
    # every position of a block is used exactly once
    cols = np.arange(R)
    p = np.array([[pos(r, c) for c in cols] for r in range(32)])
    assert np.array_equal(np.sort(p.ravel()), np.arange(32 * R))
    back = kdt.untile_partials(tiled, M)
    assert torch.equal(back, vals)


def test_bf16_lane_runs_are_contiguous():
    """In the bf16 layout the 8 values a lane holds for one column group (two
    4-column register groups) are 16 contiguous bytes, and the 64 lanes of a
    wave cover one 1 KB run."""
    R = 64
    for cg in range(R // 16):
        offs = []
        for lane in range(64):
            r, hh = lane % 32, lane // 32
            cs = [16 * cg + 8 * (i // 4) + 4 * hh + i % 4 for i in range(8)]
            ps = [_pos_bf16(r, c) for c in cs]
            assert ps == list(range(ps[0], ps[0] + 8)) and ps[0] == 512 * cg + 8 * lane
            offs.extend(ps)
        assert sorted(offs) == list(range(512 * cg, 512 * (cg + 1)))
