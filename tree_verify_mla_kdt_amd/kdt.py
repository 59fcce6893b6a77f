"""ctypes binding of libkdt.so (the C ABI in include/kdt.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the current HIP
stream.  There is no fallback: if the library is missing or a call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkdt.so")

KDT_F32, KDT_BF16 = 0, 1
ABI_VERSION = 5                       # the KDT_ABI_VERSION this binding was written for
KDT_SEQ_BAD_TREE, KDT_SEQ_BAD_LEN, KDT_SEQ_BAD_INDEX = 1, 2, 4
MAX_Q_LEN = 128

_c_i32, _c_i64, _c_p, _c_f = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float


class VerifyDesc(ctypes.Structure):
    _fields_ = [
        ("dtype", _c_i32), ("B", _c_i32), ("q_len", _c_i32), ("H", _c_i32), ("R", _c_i32), ("P", _c_i32),
        ("q_lat", _c_p), ("q_lat_sb", _c_i64), ("q_lat_st", _c_i64), ("q_lat_sh", _c_i64),
        ("q_pe", _c_p), ("q_pe_sb", _c_i64), ("q_pe_st", _c_i64), ("q_pe_sh", _c_i64),
        ("c_kv", _c_p), ("c_kv_sb", _c_i64), ("c_kv_ss", _c_i64),
        ("k_pe", _c_p), ("k_pe_sb", _c_i64), ("k_pe_ss", _c_i64),
        ("capacity", _c_i64),
        ("prefix_lens", _c_p), ("max_prefix_len", _c_i32),
        ("vis", _c_p),
        ("softmax_scale", _c_f),
        ("out", _c_p), ("out_sb", _c_i64), ("out_st", _c_i64), ("out_sh", _c_i64),
        ("lse", _c_p),
        ("seq_status", _c_p),
        ("split_keys", _c_i32), ("layout", _c_i32), ("partials_f32", _c_i32),
        ("parents", _c_p),
        ("merge_mode", _c_i32), ("merge_wait_us", _c_i32),
        ("total_prefix_len", _c_i64), ("schedule", _c_i32), ("gang_size", _c_i32),
    ]


class VerifyPlan(ctypes.Structure):
    _fields_ = [
        ("split_keys", _c_i32), ("max_splits", _c_i32), ("rows", _c_i32), ("direct", _c_i32),
        ("layout", _c_i32), ("part_dtype", _c_i32), ("part_o_offset", _c_i64), ("part_lse_offset", _c_i64),
        ("workspace_bytes", ctypes.c_size_t), ("partials_bytes", ctypes.c_size_t), ("fused_merge", _c_i32),
        ("tiles_max", _c_i32), ("counter_offset", _c_i64), ("gang_size", _c_i32), ("gangs", _c_i32),
        ("piece_units", _c_i32), ("reserved", _c_i32),
    ]


class KdtError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {code} ({status_str(code)})")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkdt.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m tree_verify_mla_kdt_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.kdt_abi_version.restype = ctypes.c_int
        L.kdt_status_str.restype = ctypes.c_char_p
        L.kdt_status_str.argtypes = [ctypes.c_int]
        L.kdt_build_visibility.argtypes = [_c_p, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_p]
        L.kdt_verify_get_plan.argtypes = [ctypes.POINTER(VerifyDesc), ctypes.POINTER(VerifyPlan)]
        L.kdt_verify_attn.argtypes = [ctypes.POINTER(VerifyDesc), _c_p, ctypes.c_size_t, _c_p]
        L.kdt_verify_partials.argtypes = [ctypes.POINTER(VerifyDesc), _c_p, ctypes.c_size_t, _c_p]
        L.kdt_verify_attn_noalloc.argtypes = [ctypes.POINTER(VerifyDesc), _c_p]
        L.kdt_merge_partials.argtypes = [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_p, _c_p, _c_i32, _c_p,
                                         _c_i32, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p]
        L.kdt_gather_accepted.argtypes = [_c_i32, _c_i32, _c_i32, _c_i32, _c_p, _c_i64, _c_i64, _c_i64, _c_i32,
                                          _c_i64, _c_p, _c_p, _c_p, _c_i32, _c_p, _c_p, _c_p]
        L.kdt_tree_accept.argtypes = [_c_p, _c_p, _c_p, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_p, _c_p]
        L.kdt_build_tree.argtypes = [_c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_p,
                                     _c_p, _c_p, _c_p, _c_p]
        L.kdt_absorb_q.argtypes = [_c_i32] * 7 + [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, ctypes.c_float,
                                                  _c_p, _c_p, _c_p]
        L.kdt_absorb_o.argtypes = [_c_i32] * 6 + [_c_p, _c_p, _c_p, _c_p]
        L.kdt_append_tree_kv.argtypes = [_c_i32] * 5 + [_c_p, _c_p, _c_p, _c_p, ctypes.c_float, _c_p, _c_i64, _c_i64,
                                                        _c_i64, _c_p, _c_p]
        for fn in ("kdt_build_visibility", "kdt_verify_get_plan", "kdt_verify_attn", "kdt_verify_attn_noalloc",
                   "kdt_verify_partials",
                   "kdt_merge_partials", "kdt_gather_accepted", "kdt_tree_accept", "kdt_build_tree",
                   "kdt_absorb_q", "kdt_absorb_o", "kdt_append_tree_kv"):
            getattr(L, fn).restype = ctypes.c_int
        if L.kdt_abi_version() != ABI_VERSION:
            raise RuntimeError("libkdt.so ABI version mismatch")
        _lib = L
    return _lib


def status_str(code: int) -> str:
    return lib().kdt_status_str(int(code)).decode()


def _check(fn: str, code: int):
    if code != 0:
        raise KdtError(fn, code)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDT_BF16
    if t.dtype == torch.float32:
        return KDT_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


# ---------------------------------------------------------------------------

def build_visibility(parents: torch.Tensor, vis=None, depth=None, seq_status=None, stream=None):
    """parents int32 [B, q] -> (vis int64 [B, q, W] holding uint64 bits, depth int32 [B, q])."""
    assert parents.dtype == torch.int32 and parents.is_contiguous() and parents.dim() == 2
    B, q = parents.shape
    W = (q + 63) // 64
    if vis is None:
        vis = torch.empty((B, q, W), dtype=torch.int64, device=parents.device)
    if depth is None:
        depth = torch.empty((B, q), dtype=torch.int32, device=parents.device)
    _check("kdt_build_visibility", lib().kdt_build_visibility(
        _ptr(parents), B, q, _ptr(vis), _ptr(depth), _ptr(seq_status), _stream(stream)))
    return vis, depth


def _verify_desc(q_lat, q_pe, c_kv, k_pe, prefix_lens, vis, softmax_scale, max_prefix_len, out, lse,
                 seq_status, split_keys, layout=0, partials_f32=False, parents=None, merge_mode=0, merge_wait_us=0,
                 total_prefix_len=0, schedule=0, gang_size=0):
    B, q, H, R = q_lat.shape
    P = q_pe.shape[-1]
    d = VerifyDesc()
    d.dtype = _dtype_code(q_lat)
    d.B, d.q_len, d.H, d.R, d.P = B, q, H, R, P
    d.q_lat = q_lat.data_ptr(); d.q_lat_sb, d.q_lat_st, d.q_lat_sh = q_lat.stride()[:3]
    d.q_pe = q_pe.data_ptr(); d.q_pe_sb, d.q_pe_st, d.q_pe_sh = q_pe.stride()[:3]
    d.c_kv = c_kv.data_ptr(); d.c_kv_sb, d.c_kv_ss = c_kv.stride()[:2]
    d.k_pe = k_pe.data_ptr(); d.k_pe_sb, d.k_pe_ss = k_pe.stride()[:2]
    d.capacity = c_kv.shape[1]
    d.prefix_lens = prefix_lens.data_ptr()
    d.max_prefix_len = int(max_prefix_len)
    d.vis = 0 if vis is None else vis.data_ptr()
    d.parents = 0 if parents is None else parents.data_ptr()
    d.softmax_scale = float(softmax_scale)
    d.out = out.data_ptr(); d.out_sb, d.out_st, d.out_sh = out.stride()[:3]
    d.lse = lse.data_ptr()
    d.seq_status = 0 if seq_status is None else seq_status.data_ptr()
    d.split_keys = int(split_keys)
    d.layout = int(layout)
    d.partials_f32 = 1 if partials_f32 else 0
    d.merge_mode = int(merge_mode)
    d.merge_wait_us = int(merge_wait_us)
    d.total_prefix_len = int(total_prefix_len)
    d.schedule = int(schedule)
    d.gang_size = int(gang_size)
    return d


def _verify_prepare(q_lat, q_pe, c_kv, k_pe, prefix_lens, vis, softmax_scale, max_prefix_len, out, lse,
                    seq_status, split_keys, layout=0, partials_f32=False, parents=None, merge_mode=0,
                    merge_wait_us=0, total_prefix_len=0, schedule=0, gang_size=0):
    for t in (q_lat, q_pe, c_kv, k_pe):
        if t.stride(-1) != 1:
            raise ValueError("innermost dimension must be contiguous")
    if not (q_lat.dtype == q_pe.dtype == c_kv.dtype == k_pe.dtype):
        raise TypeError("q_lat, q_pe, c_kv and k_pe must share one dtype")
    assert prefix_lens.dtype == torch.int32
    if vis is None:
        if parents is None:
            raise ValueError("give vis or parents")
        assert parents.dtype == torch.int32 and parents.is_contiguous() and parents.shape == q_lat.shape[:2]
    else:
        assert vis.dtype == torch.int64
    B, q, H, R = q_lat.shape
    if max_prefix_len is None:
        max_prefix_len = c_kv.shape[1] - q        # always an upper bound on a valid prefix
    if out is None:
        out = torch.empty((B, q, H, R), dtype=q_lat.dtype, device=q_lat.device)
    if lse is None:
        lse = torch.empty((B, q, H), dtype=torch.float32, device=q_lat.device)
    d = _verify_desc(q_lat, q_pe, c_kv, k_pe, prefix_lens, vis, softmax_scale, max_prefix_len, out, lse,
                     seq_status, split_keys, layout, partials_f32, parents, merge_mode, merge_wait_us,
                     total_prefix_len, schedule, gang_size)
    return d, out, lse


def verify_plan(desc: VerifyDesc) -> VerifyPlan:
    p = VerifyPlan()
    _check("kdt_verify_get_plan", lib().kdt_verify_get_plan(ctypes.byref(desc), ctypes.byref(p)))
    return p


def verify_attn(q_lat, q_pe, c_kv, k_pe, prefix_lens, vis, softmax_scale, max_prefix_len=None, out=None,
                lse=None, workspace=None, seq_status=None, split_keys=0, stream=None, layout=0, partials_f32=False,
                parents=None, merge_mode=0, merge_wait_us=0, total_prefix_len=0, schedule=0, gang_size=0):
    """Tree-verify attention.  c_kv [B, S, R] and k_pe [B, S, P] may be views of
    one fused [B, S, R+P] cache.  vis may be None when parents [B, q] int32 is
    given (the split kernel then derives the masks).  merge_mode 1 merges the
    splits inside the split kernel (when the launch fits the device); a
    caller-given workspace must then have been allocated zeroed (its merge
    state words; every call leaves their counts at zero).  Without a workspace
    a zeroed one is allocated per call.  total_prefix_len (the sum of the
    prefix lengths, 0 = unknown) sizes the launch; schedule 1 forces splits,
    2 the balanced schedule (gang_size row tiles per gang, 0 = the library's
    choice).  Returns
    (out [B, q, H, R], lse [B, q, H])."""
    d, out, lse = _verify_prepare(q_lat, q_pe, c_kv, k_pe, prefix_lens, vis, softmax_scale, max_prefix_len,
                                  out, lse, seq_status, split_keys, layout, partials_f32, parents, merge_mode,
                                  merge_wait_us, total_prefix_len, schedule, gang_size)
    p = verify_plan(d)
    if p.workspace_bytes and (workspace is None or workspace.numel() * workspace.element_size() < p.workspace_bytes):
        workspace = torch.zeros(p.workspace_bytes, dtype=torch.uint8, device=q_lat.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("kdt_verify_attn", lib().kdt_verify_attn(ctypes.byref(d), _ptr(workspace), ws_bytes, _stream(stream)))
    return out, lse


NOALLOC_MAX_WORKSPACE = 32 << 20              # KDT_NOALLOC_MAX_WORKSPACE


def verify_attn_noalloc(q_lat, q_pe, c_kv, k_pe, prefix_lens, vis, softmax_scale, max_prefix_len=None, out=None,
                        lse=None, seq_status=None, split_keys=0, stream=None, layout=0, partials_f32=False,
                        parents=None, total_prefix_len=0, schedule=0, gang_size=0):
    """kdt_verify_attn_noalloc: the same as verify_attn, with the library's own
    fixed device workspace (no allocation; calls on one GPU must not
    overlap).  out and lse should be given when nothing may be allocated."""
    d, out, lse = _verify_prepare(q_lat, q_pe, c_kv, k_pe, prefix_lens, vis, softmax_scale, max_prefix_len,
                                  out, lse, seq_status, split_keys, layout, partials_f32, parents,
                                  total_prefix_len=total_prefix_len, schedule=schedule, gang_size=gang_size)
    _check("kdt_verify_attn_noalloc", lib().kdt_verify_attn_noalloc(ctypes.byref(d), _stream(stream)))
    return out, lse


def partial_blocks(rows: int) -> int:
    """Number of 32-row blocks of the partial layout for q_len*H = rows."""
    return (rows + 31) // 32


def untile_partials(part_o, rows: int):
    """Row-major view of tiled partials: [B, S, NBLK, 32*R] -> [B, S, rows, R].

    In the tiled layout, column c of row r of a 32-row block sits at
    256*(c//8) + 128*((c//4)%2) + 4*r + c%4 (float32) or at
    512*(c//16) + 8*(r + 32*((c//4)%2)) + 4*((c//8)%2) + c%4 (bf16): the
    order of a 32x32 matrix-core accumulator."""
    B, S, nblk, w = part_o.shape
    R = w // 32
    if part_o.dtype == torch.bfloat16:
        t = part_o.reshape(B, S, nblk, R // 16, 2, 32, 2, 4).permute(0, 1, 2, 5, 3, 6, 4, 7)
    else:
        t = part_o.reshape(B, S, nblk, R // 8, 2, 32, 4).permute(0, 1, 2, 5, 3, 4, 6)
    return t.reshape(B, S, nblk * 32, R)[:, :, :rows]


def tile_partials(rows_major):
    """Inverse of untile_partials: [B, S, rows, R] -> contiguous [B, S, NBLK, 32*R]
    in the encoding of rows_major's dtype (padding rows zero)."""
    B, S, M, R = rows_major.shape
    nblk = partial_blocks(M)
    pad = rows_major.new_zeros((B, S, nblk * 32, R))
    pad[:, :, :M] = rows_major
    if rows_major.dtype == torch.bfloat16:
        t = pad.reshape(B, S, nblk, 32, R // 16, 2, 2, 4).permute(0, 1, 2, 4, 6, 3, 5, 7)
    else:
        t = pad.reshape(B, S, nblk, 32, R // 8, 2, 4).permute(0, 1, 2, 4, 5, 3, 6)
    return t.contiguous().reshape(B, S, nblk, 32 * R)


def verify_partials(q_lat, q_pe, c_kv, k_pe, prefix_lens, vis, softmax_scale, max_prefix_len=None,
                    workspace=None, seq_status=None, split_keys=0, stream=None, layout=0, partials_f32=False,
                    parents=None, total_prefix_len=0, schedule=0, gang_size=0):
    """Split stage only.  Returns (part_o, part_lse, plan): part_o
    [B, S, NBLK, 32*R] in the tiled layout (see untile_partials), bf16 for
    bf16 inputs unless partials_f32, else float32; part_lse float32 [B, S, q*H]."""
    d, _, _ = _verify_prepare(q_lat, q_pe, c_kv, k_pe, prefix_lens, vis, softmax_scale, max_prefix_len,
                              None, None, seq_status, split_keys, layout, partials_f32, parents,
                              total_prefix_len=total_prefix_len, schedule=schedule, gang_size=gang_size)
    p = verify_plan(d)
    B, R, M, S = q_lat.shape[0], q_lat.shape[3], p.rows, p.max_splits
    need = max(int(p.partials_bytes), 1)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_lat.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("kdt_verify_partials", lib().kdt_verify_partials(ctypes.byref(d), _ptr(workspace), ws_bytes,
                                                           _stream(stream)))
    nblk = partial_blocks(M)
    n_o = B * S * nblk * 32 * R
    pdt = torch.bfloat16 if p.part_dtype == KDT_BF16 else torch.float32
    es = 2 if p.part_dtype == KDT_BF16 else 4
    part_o = workspace[p.part_o_offset:p.part_o_offset + n_o * es].view(pdt).view(B, S, nblk, 32 * R)
    part_lse = workspace[p.part_lse_offset:p.part_lse_offset + B * S * M * 4].view(torch.float32).view(B, S, M)
    return part_o, part_lse, p


def merge_partials(part_o, part_lse, q_len, H, out_dtype, prefix_lens=None, split_keys=0, out=None, lse=None,
                   stream=None):
    """part_o float32 or bf16 [B, S, NBLK, 32*R] (tiled), part_lse float32
    [B, S, q*H] -> (out [B, q, H, R], lse [B, q, H])."""
    B, S, nblk, w = part_o.shape
    R = w // 32
    assert nblk == partial_blocks(q_len * H) and part_lse.shape == (B, S, q_len * H)
    assert part_o.is_contiguous() and part_lse.is_contiguous()
    if out is None:
        out = torch.empty((B, q_len, H, R), dtype=out_dtype, device=part_o.device)
    if lse is None:
        lse = torch.empty((B, q_len, H), dtype=torch.float32, device=part_o.device)
    code = KDT_BF16 if out.dtype == torch.bfloat16 else KDT_F32
    sb, st, sh = out.stride()[:3]
    _check("kdt_merge_partials", lib().kdt_merge_partials(
        code, B, q_len, H, R, KDT_BF16 if part_o.dtype == torch.bfloat16 else KDT_F32, _ptr(part_o), _ptr(part_lse), S, _ptr(prefix_lens), int(split_keys), _ptr(out),
        sb, st, sh, _ptr(lse), _stream(stream)))
    return out, lse


def gather_accepted(cache, prefix_lens, accepted, n_accepted, q_len, row_elems=None, num_layers=1,
                    layer_stride=0, new_prefix_lens=None, seq_status=None, stream=None):
    """In-place accepted-path gather on cache [B, S, C] (or the layer-0 view of
    a [layers, B, S, C] cache with layer_stride in elements)."""
    assert accepted.dtype == torch.int32 and n_accepted.dtype == torch.int32 and accepted.is_contiguous()
    B = cache.shape[0]
    if row_elems is None:
        row_elems = cache.shape[2]
    sb, ss = cache.stride()[:2]
    _check("kdt_gather_accepted", lib().kdt_gather_accepted(
        _dtype_code(cache), B, int(q_len), int(row_elems), _ptr(cache), sb, ss, cache.shape[1], int(num_layers),
        int(layer_stride), _ptr(prefix_lens), _ptr(accepted), _ptr(n_accepted), accepted.shape[1],
        _ptr(new_prefix_lens), _ptr(seq_status), _stream(stream)))
    return cache


def tree_accept(parents, tokens, target_pred, accepted=None, n_accepted=None, bonus=None, seq_status=None,
                stream=None):
    """Greedy tree acceptance: int32 [B, q] parents / tokens / target_pred ->
    (accepted int32 [B, q] with -1 past the path, n_accepted int32 [B], bonus int32 [B])."""
    for t in (parents, tokens, target_pred):
        assert t.dtype == torch.int32 and t.is_contiguous() and t.dim() == 2 and t.shape == parents.shape
    B, q = parents.shape
    dev = parents.device
    if accepted is None:
        accepted = torch.empty((B, q), dtype=torch.int32, device=dev)
    if n_accepted is None:
        n_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if bonus is None:
        bonus = torch.empty((B,), dtype=torch.int32, device=dev)
    _check("kdt_tree_accept", lib().kdt_tree_accept(
        _ptr(parents), _ptr(tokens), _ptr(target_pred), B, q, _ptr(accepted), _ptr(n_accepted), _ptr(bonus),
        _ptr(seq_status), _stream(stream)))
    return accepted, n_accepted, bonus


def build_tree(topk_tokens, topk_logprobs, root_tokens, q_len, with_links=True, stream=None):
    """Best-first draft tree: int32 [B, D, K] tokens, float32 [B, D, K]
    log-probabilities (best first), int32 [B] root tokens -> dict of device
    tensors parents / tokens / depth (int32 [B, q]), logw (float64 [B, q]),
    first_child / next_sibling (int32 [B, q], if with_links), n_nodes (int32 [B])."""
    assert topk_tokens.dtype == torch.int32 and topk_logprobs.dtype == torch.float32
    assert root_tokens.dtype == torch.int32
    for t in (topk_tokens, topk_logprobs, root_tokens):
        assert t.is_contiguous()
    B, D, K = topk_tokens.shape
    assert topk_logprobs.shape == (B, D, K) and root_tokens.shape == (B,)
    dev = topk_tokens.device
    out = {k: torch.empty((B, q_len), dtype=torch.int32, device=dev) for k in ("parents", "tokens", "depth")}
    out["logw"] = torch.empty((B, q_len), dtype=torch.float64, device=dev)
    if with_links:
        out["first_child"] = torch.empty((B, q_len), dtype=torch.int32, device=dev)
        out["next_sibling"] = torch.empty((B, q_len), dtype=torch.int32, device=dev)
    out["n_nodes"] = torch.empty((B,), dtype=torch.int32, device=dev)
    _check("kdt_build_tree", lib().kdt_build_tree(
        _ptr(topk_tokens), _ptr(topk_logprobs), _ptr(root_tokens), B, D, K, int(q_len), _ptr(out["parents"]),
        _ptr(out["tokens"]), _ptr(out["depth"]), _ptr(out["logw"]), _ptr(out.get("first_child")),
        _ptr(out.get("next_sibling")), _ptr(out["n_nodes"]), _stream(stream)))
    return out


def absorb_q(q, w_kc_t, prefix_lens, depth, dn, rope_theta, q_lat=None, q_pe=None, stream=None):
    """Query split + key absorb + rotary embedding at L + depth.
    q bf16 [B, T, H, dn + P] (innermost contiguous), w_kc_t bf16 [H, R, dn],
    prefix_lens int32 [B], depth int32 [B, T] -> (q_lat [B, T, H, R], q_pe [B, T, H, P])."""
    assert q.dtype == torch.bfloat16 and w_kc_t.dtype == torch.bfloat16 and w_kc_t.is_contiguous()
    assert q.stride(-1) == 1 and depth.dtype == torch.int32 and depth.is_contiguous()
    B, T, H, E = q.shape
    P = E - dn
    R = w_kc_t.shape[1]
    if q_lat is None:
        q_lat = torch.empty((B, T, H, R), dtype=torch.bfloat16, device=q.device)
    if q_pe is None:
        q_pe = torch.empty((B, T, H, P), dtype=torch.bfloat16, device=q.device)
    sb, st, sh = q.stride()[:3]
    _check("kdt_absorb_q", lib().kdt_absorb_q(
        KDT_BF16, B, T, H, int(dn), P, R, _ptr(q), sb, st, sh, _ptr(w_kc_t), _ptr(prefix_lens), _ptr(depth),
        float(rope_theta), _ptr(q_lat), _ptr(q_pe), _stream(stream)))
    return q_lat, q_pe


def absorb_o(o_lat, w_vc, o=None, stream=None):
    """Value absorb: o_lat bf16 [B, T, H, R], w_vc bf16 [H, dv, R] -> o [B, T, H, dv]."""
    assert o_lat.dtype == torch.bfloat16 and o_lat.is_contiguous() and w_vc.is_contiguous()
    B, T, H, R = o_lat.shape
    dv = w_vc.shape[1]
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=o_lat.device)
    _check("kdt_absorb_o", lib().kdt_absorb_o(KDT_BF16, B, T, H, R, dv, _ptr(o_lat), _ptr(w_vc), _ptr(o),
                                              _stream(stream)))
    return o


def append_tree_kv(cache, c_kv_new, k_rope_new, prefix_lens, depth, rope_theta, seq_status=None, stream=None):
    """Cache append of the tree tokens into cache [B, S, R + P] (in place)."""
    assert cache.dtype == torch.bfloat16 and c_kv_new.is_contiguous() and k_rope_new.is_contiguous()
    B, T, R = c_kv_new.shape
    P = k_rope_new.shape[-1]
    sb, ss = cache.stride()[:2]
    _check("kdt_append_tree_kv", lib().kdt_append_tree_kv(
        KDT_BF16, B, T, R, P, _ptr(c_kv_new), _ptr(k_rope_new), _ptr(prefix_lens), _ptr(depth),
        float(rope_theta), _ptr(cache), sb, ss, cache.shape[1], _ptr(seq_status), _stream(stream)))
    return cache


def softmax_scale_for(R: int, P: int) -> float:
    return 1.0 / math.sqrt(R + P)
