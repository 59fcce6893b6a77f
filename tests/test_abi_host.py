"""The C ABI on the CPU: the library loads, exports every symbol that
include/kdt.h declares, and its host-side checks and planning work without
launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest

from tree_verify_mla_kdt_amd import kdt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kdt.h")
FAKE = 0x10000     # never dereferenced: these calls fail validation before any launch


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kdt_[a-z_]+)\s*\(", text)))


def test_header_symbols_are_exported():
    names = declared_functions()
    assert "kdt_verify_attn" in names and "kdt_gather_accepted" in names and "kdt_build_visibility" in names
    L = kdt.lib()
    for n in names:
        assert hasattr(L, n), f"libkdt.so does not export {n}"


def test_version_and_status_strings():
    assert kdt.lib().kdt_abi_version() == kdt.ABI_VERSION == 5
    for code in range(5):
        assert kdt.status_str(code)
    assert kdt.status_str(99) == "unknown status"


def _desc(**kw):
    d = kdt.VerifyDesc()
    d.dtype, d.B, d.q_len, d.H, d.R, d.P = 1, 1, 65, 16, 512, 64
    for f in ("q_lat", "q_pe", "c_kv", "k_pe", "prefix_lens", "vis", "out", "lse"):
        setattr(d, f, FAKE)
    d.q_lat_sb, d.q_lat_st, d.q_lat_sh = 65 * 16 * 512, 16 * 512, 512
    d.q_pe_sb, d.q_pe_st, d.q_pe_sh = 65 * 16 * 64, 16 * 64, 64
    d.c_kv_sb, d.c_kv_ss, d.k_pe_sb, d.k_pe_ss = 4224 * 576, 576, 4224 * 576, 576
    d.capacity, d.max_prefix_len, d.softmax_scale = 4224, 4096, 576 ** -0.5
    d.out_sb, d.out_st, d.out_sh = 65 * 16 * 512, 16 * 512, 512
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _plan(d):
    p = kdt.VerifyPlan()
    rc = kdt.lib().kdt_verify_get_plan(ctypes.byref(d), ctypes.byref(p))
    return rc, p


def test_plan_sizes_and_layout():
    rc, p = _plan(_desc())
    assert rc == 0
    M = 65 * 16
    assert p.rows == M
    assert p.split_keys % 32 == 0 and p.split_keys >= 32
    assert p.max_splits == -(-(4096 + 65) // p.split_keys)
    assert p.direct == (1 if p.max_splits == 1 else 0)
    nblk = -(-M // 32)
    assert p.part_dtype == kdt.KDT_BF16            # bf16 inputs: bf16 partials unless asked otherwise
    assert p.part_lse_offset >= 1 * p.max_splits * nblk * 32 * 512 * 2 and p.part_lse_offset % 256 == 0
    assert p.partials_bytes == p.part_lse_offset + p.max_splits * M * 4
    # merge state words (one int32 per row tile) after the partials, 256-byte aligned
    n_rt = -(-M // (128 if p.layout == 1 else 64))
    assert p.counter_offset % 256 == 0 and p.counter_offset >= p.partials_bytes
    assert p.workspace_bytes == p.counter_offset + n_rt * 4
    assert p.fused_merge == 0                      # the separate merge kernel is the default
    rc, ps = _plan(_desc(merge_mode=1, split_keys=p.split_keys, layout=p.layout))
    assert rc == 0 and ps.partials_bytes == p.partials_bytes and ps.workspace_bytes == p.workspace_bytes
    assert _plan(_desc(merge_mode=2))[0] == 1
    rc, p32 = _plan(_desc(partials_f32=1, split_keys=p.split_keys))
    assert rc == 0 and p32.part_dtype == kdt.KDT_F32 and p32.max_splits == p.max_splits
    assert p32.part_lse_offset >= p.max_splits * nblk * 32 * 512 * 4
    assert _plan(_desc(partials_f32=2))[0] == 1
    rc, p = _plan(_desc(split_keys=128))
    assert rc == 0 and p.split_keys == 128 and p.max_splits == 33
    # a single split: no workspace for kdt_verify_attn, partials still sized
    rc, p = _plan(_desc(split_keys=8192))
    assert rc == 0 and p.direct == 1 and p.max_splits == 1
    assert p.workspace_bytes == 0 and p.fused_merge == 0
    assert p.partials_bytes == p.part_lse_offset + M * 4


@pytest.mark.parametrize("field,value,code", [
    ("q_lat", 0, 1), ("lse", 0, 1), ("B", 0, 1), ("H", -1, 1),
    ("capacity", 4100, 1),                 # below max_prefix_len + q_len
    ("split_keys", 100, 1),                # not a multiple of 32 (the key tile)
    ("split_keys", 48, 1),
    ("softmax_scale", 0.0, 1),
    ("q_len", 129, 2),                     # beyond two mask words
    ("R", 256, 2), ("dtype", 7, 2),
    ("q_lat_sh", 500, 2),                  # stride not 16-byte aligned
    ("q_lat", FAKE + 2, 2),                # pointer not 16-byte aligned
])
def test_plan_rejects_bad_descriptors(field, value, code):
    kw = {field: value}
    if field == "q_len":
        kw["max_prefix_len"] = 1000        # keep the capacity check satisfied
    rc, _ = _plan(_desc(**kw))
    assert rc == code


def test_split_rows_fit_32bit_offsets():
    """The split kernel addresses a split's cache rows by 32-bit byte offsets
    from its first row, so split_keys rows of either region must span less
    than 2^31 bytes: a larger forced split is unsupported, and the automatic
    plan stays below the limit."""
    row_bytes = 576 * 2                                   # bf16 rows of R + P = 576
    limit = (2 ** 31 - 1) // row_bytes // 32 * 32
    rc, p = _plan(_desc(split_keys=limit))
    assert rc == 0 and p.split_keys == limit
    assert _plan(_desc(split_keys=limit + 32))[0] == 2
    # a 4M-key prefix: the library's choice splits it below the limit
    rc, p = _plan(_desc(max_prefix_len=4_000_000, capacity=4_000_065))
    assert rc == 0 and 0 < p.split_keys <= limit and p.max_splits >= 3
    # a 32 MB row stride leaves one 32-key tile per split; 64 MB none (32 rows
    # of it are exactly 2^31 bytes)
    big = 1 << 24                                         # elements per row
    rc, p = _plan(_desc(c_kv_ss=big, k_pe_ss=big, c_kv_sb=big * 4224, k_pe_sb=big * 4224))
    assert rc == 0 and p.split_keys == 32
    assert _plan(_desc(c_kv_ss=2 * big, k_pe_ss=64, c_kv_sb=2 * big * 4224))[0] == 2


def test_balanced_schedule_plan():
    """The balanced schedule on request: one workgroup per compute unit (the
    host query falls back to 256 without a device), gangs of gang_size row
    tiles, at least two partial slots per row, and the balance rule's bound on
    slots per stream (the longest stream over ranges of A key tiles)."""
    rc, p = _plan(_desc(schedule=2))
    assert rc == 0 and p.gang_size > 0 and p.gangs == 256 // p.gang_size and p.layout in (1, 2)
    assert p.direct == 0 and p.tiles_max == 0 and p.fused_merge == 0 and p.max_splits >= 2
    T = -(-(4096 + 65) // 32)
    n_rt = -(-(65 * 16) // (128 if p.layout == 1 else 64))
    assert p.piece_units > 0
    U = -(-n_rt // p.gang_size) * (T + p.piece_units)
    A = -(-U // p.gangs)
    assert p.max_splits == max(2, -(-T // A) + 1)
    for g in (1, 3, 9):
        rc, p = _plan(_desc(schedule=2, gang_size=g, layout=1))
        assert rc == 0 and p.gang_size == g and p.gangs == 256 // g
    assert _plan(_desc(schedule=2, gang_size=10, layout=1))[0] == 1     # more than the 9 row tiles
    assert _plan(_desc(schedule=2, split_keys=256))[0] == 1             # the balanced schedule sizes its own ranges
    assert _plan(_desc(schedule=3))[0] == 1
    assert _plan(_desc(gang_size=-1))[0] == 1
    assert _plan(_desc(schedule=2, layout=4))[0] == 2                   # layouts 1 and 2 only
    # units counted in 32 bits: 4096 sequences of up to 20M keys are too many
    assert _plan(_desc(schedule=2, B=4096, max_prefix_len=20_000_000, capacity=20_000_065))[0] == 2
    rc, p = _plan(_desc(B=4096, max_prefix_len=20_000_000, capacity=20_000_065))
    assert rc == 0 and p.gang_size == 0
    rc, p = _plan(_desc(schedule=1))
    assert rc == 0 and p.gang_size == 0


def test_masks_or_parents_required():
    assert _plan(_desc(vis=0))[0] == 1                 # neither masks nor parents
    rc, _ = _plan(_desc(vis=0, parents=FAKE))          # masks derived from parents
    assert rc == 0


def test_fp32_large_rank_is_unsupported():
    rc, _ = _plan(_desc(dtype=0))
    assert rc == 2
    d = _desc(dtype=0, R=64, P=16, q_lat_sh=64, q_lat_st=16 * 64, q_lat_sb=65 * 16 * 64,
              q_pe_sh=16, q_pe_st=16 * 16, q_pe_sb=65 * 16 * 16, c_kv_ss=80, k_pe_ss=80,
              c_kv_sb=4224 * 80, k_pe_sb=4224 * 80, out_sh=64, out_st=16 * 64, out_sb=65 * 16 * 64)
    rc, p = _plan(d)
    assert rc == 0


def test_verify_needs_workspace_when_split():
    d = _desc()
    rc = kdt.lib().kdt_verify_attn(ctypes.byref(d), None, 0, None)
    assert rc == 3


def test_visibility_gather_accept_and_tree_argument_checks():
    L = kdt.lib()
    assert L.kdt_build_visibility(None, 1, 9, FAKE, None, None, None) == 1
    assert L.kdt_build_visibility(FAKE, 0, 9, FAKE, None, None, None) == 1
    assert L.kdt_build_visibility(FAKE, 1, 129, FAKE, None, None, None) == 2
    g = L.kdt_gather_accepted
    # dtype, B, q, row_elems, cache, sb, ss, capacity, layers, layer_stride, pl, acc, nacc, max_acc, npl, st, stream
    assert g(1, 1, 9, 576, None, 0, 576, 64, 1, 0, FAKE, FAKE, FAKE, 9, None, None, None) == 1
    assert g(1, 1, 9, 576, FAKE, 0, 576, 64, 1, 0, FAKE, FAKE, FAKE, 10, None, None, None) == 1   # max_acc > q
    assert g(1, 1, 9, 576, FAKE, 0, 576, 64, 1, 0, FAKE, FAKE, FAKE, 9, FAKE, None, None) == 1    # npl aliases pl
    assert g(5, 1, 9, 576, FAKE, 0, 576, 64, 1, 0, FAKE, FAKE, FAKE, 9, None, None, None) == 2    # dtype
    assert g(1, 1, 200, 576, FAKE, 0, 576, 256, 1, 0, FAKE, FAKE, FAKE, 9, None, None, None) == 2
    m = L.kdt_merge_partials
    assert m(1, 1, 9, 4, 512, 0, None, FAKE, 2, None, 0, FAKE, 0, 0, 0, FAKE, None) == 1
    assert m(1, 1, 9, 4, 512, 0, FAKE, FAKE, 2, None, 64, FAKE, 0, 0, 0, FAKE, None) == 1        # needs prefix_lens
    assert m(1, 1, 9, 4, 36, 0, FAKE, FAKE, 2, None, 0, FAKE, 0, 0, 0, FAKE, None) == 2          # R % 8
    assert m(1, 1, 9, 4, 40, 1, FAKE, FAKE, 2, None, 0, FAKE, 0, 0, 0, FAKE, None) == 2          # bf16 partials: R % 16
    assert m(1, 1, 9, 4, 512, 2, FAKE, FAKE, 2, None, 0, FAKE, 0, 0, 0, FAKE, None) == 2         # partial dtype
    a = L.kdt_tree_accept
    # parents, tokens, target_pred, B, q, accepted, n_accepted, bonus, seq_status, stream
    assert a(None, FAKE, FAKE, 1, 9, FAKE, FAKE, None, None, None) == 1
    assert a(FAKE, FAKE, FAKE, 1, 9, None, FAKE, None, None, None) == 1
    assert a(FAKE, FAKE, FAKE, 0, 9, FAKE, FAKE, None, None, None) == 1
    assert a(FAKE, FAKE, FAKE, 1, 0, FAKE, FAKE, None, None, None) == 1
    assert a(FAKE, FAKE, FAKE, 1, 129, FAKE, FAKE, None, None, None) == 2
    t = L.kdt_build_tree
    # topk_tokens, topk_logprobs, roots, B, D, K, q, parents, tokens, depth, logw, first, next, n, stream
    assert t(None, FAKE, FAKE, 1, 4, 4, 9, FAKE, FAKE, FAKE, None, None, None, None, None) == 1
    assert t(FAKE, FAKE, FAKE, 1, 4, 4, 9, FAKE, None, FAKE, None, None, None, None, None) == 1
    assert t(FAKE, FAKE, FAKE, 1, 0, 4, 9, FAKE, FAKE, FAKE, None, None, None, None, None) == 1
    assert t(FAKE, FAKE, FAKE, 1, 4, 0, 9, FAKE, FAKE, FAKE, None, None, None, None, None) == 1
    assert t(FAKE, FAKE, FAKE, 1, 4, 4, 129, FAKE, FAKE, FAKE, None, None, None, None, None) == 2
    assert t(FAKE, FAKE, FAKE, 1, 4, 65, 65, FAKE, FAKE, FAKE, None, None, None, None, None) == 2
    aq = L.kdt_absorb_q
    # dtype, B, T, H, dn, P, R, q, sb, st, sh, w, pl, depth, theta, q_lat, q_pe, stream
    assert aq(1, 1, 9, 16, 128, 64, 512, None, 0, 0, 0, FAKE, FAKE, FAKE, 1e4, FAKE, FAKE, None) == 1
    assert aq(1, 1, 9, 16, 128, 64, 512, FAKE, 0, 0, 0, FAKE, FAKE, FAKE, 0.5, FAKE, FAKE, None) == 1
    assert aq(0, 1, 9, 16, 128, 64, 512, FAKE, 0, 0, 0, FAKE, FAKE, FAKE, 1e4, FAKE, FAKE, None) == 2  # fp32
    assert aq(1, 1, 9, 16, 128, 63, 512, FAKE, 0, 0, 0, FAKE, FAKE, FAKE, 1e4, FAKE, FAKE, None) == 2  # odd P
    assert aq(1, 1, 9, 16, 128, 64, 512, FAKE, 3, 0, 0, FAKE, FAKE, FAKE, 1e4, FAKE, FAKE, None) == 2  # stride
    ao = L.kdt_absorb_o
    assert ao(1, 1, 9, 16, 512, 128, None, FAKE, FAKE, None) == 1
    assert ao(1, 1, 9, 16, 512, 128, FAKE + 2, FAKE, FAKE, None) == 2                            # alignment
    ap = L.kdt_append_tree_kv
    assert ap(1, 1, 9, 512, 64, FAKE, FAKE, FAKE, FAKE, 1e4, None, 0, 576, 64, None, None) == 1
    assert ap(1, 1, 9, 512, 64, FAKE, FAKE, FAKE, FAKE, 1e4, FAKE, 0, 500, 64, None, None) == 1   # row too short


def test_auto_split_counts_follow_the_launch_model():
    # batch 64 x 3 row tiles already fill the chip: one split, no merge
    rc, p = _plan(_desc(B=64, q_len=17, max_prefix_len=2048, capacity=2048 + 17))
    assert rc == 0 and p.max_splits == 1 and p.direct == 1
    # batch 4 x 33 row tiles of a 32K prefix: several splits (more than two,
    # so the grid does not end with a nearly empty second round)
    rc, p = _plan(_desc(B=4, H=64, max_prefix_len=32768, capacity=32768 + 65))
    assert rc == 0 and p.max_splits > 2


def test_partial_tiling_round_trip():
    import torch
    rng = np.random.default_rng(3)
    for M, R in ((1040, 512), (21, 64), (32, 64)):
        x = torch.from_numpy(rng.standard_normal((2, 3, M, R)).astype(np.float32))
        t = kdt.tile_partials(x)
        assert t.shape == (2, 3, kdt.partial_blocks(M), 32 * R)
        assert torch.equal(kdt.untile_partials(t, M), x)
        # spot-check the documented position of (m, c)
        m, c = M - 1, R - 3
        flat = t[1, 2, m // 32]
        assert flat[256 * (c // 8) + 128 * ((c // 4) % 2) + 4 * (m % 32) + c % 4] == x[1, 2, m, c]


def test_layout_forcing_and_validation():
    for layout in (1, 2):
        rc, p = _plan(_desc(layout=layout))
        assert rc == 0 and p.layout == layout
        rows = 128 if layout == 1 else 64
        assert p.rows == 65 * 16 and rows in (64, 128)
    rc, p = _plan(_desc())
    assert rc == 0 and p.layout in (1, 2, 4)           # the planner never picks layout 3
    rc, p = _plan(_desc(R=64, P=16, q_lat_sh=64, q_lat_st=16 * 64, q_lat_sb=65 * 16 * 64,
                        q_pe_sh=16, q_pe_st=16 * 16, q_pe_sb=65 * 16 * 16, c_kv_ss=80, k_pe_ss=80,
                        c_kv_sb=4224 * 80, k_pe_sb=4224 * 80, out_sh=64, out_st=16 * 64, out_sb=65 * 16 * 64))
    assert rc == 0 and p.layout in (1, 2)              # layout 4 only for the rank-512 shape
    rc, p = _plan(_desc(layout=3))            # depth-split pairs: bf16, R = 512, P = 64
    assert rc == 0 and p.layout == 3
    rc, p = _plan(_desc(layout=3, R=64, P=16))
    assert rc == 2
    rc, p = _plan(_desc(layout=4))            # two key streams: bf16, R = 512, P = 64
    assert rc == 0 and p.layout == 4
    rc, p = _plan(_desc(layout=4, R=64, P=16))
    assert rc == 2
    rc, p = _plan(_desc(layout=5))
    assert rc == 1
    rc, p = _plan(_desc(layout=-1))
    assert rc == 1
    # AR decoding (64 rows) plans a 64-row layout (two key streams at rank 512)
    rc, p = _plan(_desc(q_len=1, H=64, max_prefix_len=32768, capacity=32769))
    assert rc == 0 and p.layout == 4
