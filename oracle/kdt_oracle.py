"""CPU oracle for tree-verify MLA-absorb attention (test infrastructure only).

This module is the correctness reference for the HIP library.  It is plain,
slow and written to be checked by eye: float64 numpy, one sequence at a time,
no blocking, no fusion.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path never does.
It shares no code with the HIP path (the only common module is the seeded input
generator, which holds no attention arithmetic).

Pages cited (titles of the four pages; sections in quotes):
  [Checkpoint]   "The Checkpoint: Committing a Working Native DDTree Engine"
  [Milestone]    "The Milestone Commit: Cementing a Native DDTree Inference Engine"
  [Final]        "The Final Commit: Cementing a Native DDTree Inference Engine for Kimi K2.6"

What is computed, and where it comes from:
  * Visibility: each tree node's ancestor-or-self bitmask, built as
    mask(node) = mask(parent) | bit(node), packed into 64-bit words with two
    words covering up to 65 nodes [Milestone, "The Reasoning Behind the
    Architecture", ancestor-bitmask visibility].
  * Verify attention: the q_len = 1 + drafts tree tokens attend over the
    cached prefix (all visible) followed by the tree itself (visible iff the
    key node is an ancestor-or-self of the query node): mask = [ones |
    visibility], prefix = cache length, and AR decoding is the q_len = 1 case
    [Checkpoint, "The Message", KV-cache scheme].  Scores are in the absorbed
    (latent) form: the query has been multiplied by w_kc upstream, so the
    score of key j is scale * (q_lat . c_kv[j] + q_pe . k_pe[j]) and the
    output is the latent context sum_j softmax_j * c_kv[j]; w_vc is applied
    downstream [Final, "Input Knowledge Required", MLA absorb form;
    Checkpoint, "The Message", absorb_qk/vc].  The per-row log-sum-exp is
    returned beside it (natural log, scale included).
  * Partial merge: attention over a key set split into chunks recombines from
    per-chunk (normalised output, log-sum-exp) pairs by the log-sum-exp
    identity.  The pages do not describe this step; it is the plain identity
    that makes split-prefix attention exact.
  * Accepted-path gather: after acceptance, the accepted path's latents are
    gathered into the rows directly after the prefix ("after accept gather
    accepted-path latents", post-verify compaction) [Checkpoint, "The
    Message"].
  * Greedy tree accept: the engine verifies the tree and accepts a prefix of
    it greedily, which must reproduce autoregressive greedy decoding
    [Final, "Input Knowledge Required"; Checkpoint, "The Message",
    tree_accept and the greedy-exact invariant].  From the root, the walk
    moves to a child whose draft token equals the target's greedy prediction
    at the current node, while one exists; the prediction at the last
    accepted node is the bonus token.  Walks are bounded by the tree size,
    the safety bound of [Milestone, "Mistakes and Incorrect Assumptions"].
  * Best-first tree build: the draft tree is built best-first from the
    drafter's top-k candidates per draft position, with a heap, accumulating
    log-probabilities in double precision; it yields the parent pointers
    (which the visibility consumes) and a first-child / next-sibling encoding
    whose sibling lists run in order of log-probability [Milestone, "The
    Context: Why This Commit Exists", "The Reasoning Behind the Architecture";
    Final, "Input Knowledge Required", best-first from top-k logits].

  * Around the verify: the query projection of a tree token is split into
    its non-positional part and its rotary part (split_q); the first is
    absorbed into the latent space with the per-head key up-projection w_kc
    (absorb_qk), the second gets NeoX rotary embedding at position L + depth;
    the tree tokens' latents and rotary keys are appended to the cache at
    rows L + t (the key again rotated at L + depth); after the verify the
    latent output is mapped back per head with w_vc (absorb_vc)
    [Checkpoint, "The Message": split_q, absorb_qk/vc, rope, cache append,
    positions L + depth; Final, "Input Knowledge Required", absorb form].

Readings where the pages are silent (each also listed in the design notes):
  * Tree node t's latents sit in cache row L_b + t (node order); its position
    L_b + depth(t) only matters to RoPE, which happens upstream.
  * Parents are int32 with parent[0] = -1 and 0 <= parent[i] < i; anything
    else is rejected here (the GPU side flags it per sequence instead).
  * Bits at or above q_len in the last word are zero.
  * The gather reads every source row before writing any destination row.
  * Accept: when several children of a node carry the predicted token, the
    lowest-index child (the earliest in best-first order) is taken; the
    accepted list starts with the root (node 0), so it feeds the gather
    directly.
  * Tree build: the drafter gives, for each draft position d = 1..D, its K
    best tokens with log-probabilities sorted best first (one list per
    position, shared by every node at depth d - 1: a block drafter predicts
    positions, not paths).  The root (node 0, the verified token) has logw 0;
    the child of rank j of a node at depth d - 1 has logw = logw(node) +
    logprob[d][j].  This is a plain heap: when a node is created (the root
    first) all K of its children go on the heap, best rank first, and nodes
    are created by popping the heap until the budget of q nodes is reached or
    the heap is empty.  Equal logw: the candidate pushed earlier wins, i.e.
    the child of the earlier created parent, then the lower rank.  Budget
    slots left over are padding: a child of the root with token -1 (no
    prediction matches it), depth 1, logw -inf.
  * Rotary embedding (NeoX form): for i < P/2 the pair (x[i], x[i + P/2]) is
    rotated by pos * theta^(-2i/P); theta is a parameter (the pages name
    YaRN for the real model as a later swap, so plain NeoX is built here).
  * Weight layouts: w_kc is given transposed per head, [H, R, dn] (row r
    holds the dn weights of latent r), and w_vc as [H, dv, R]; then both
    absorbs read each weight row contiguously along the contraction.

Parity status: every function here is pinned by CPU tests against closed
forms, brute force, library routines or invariants; none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np


# ----------------------------------------------------------------------------
# Visibility  [Milestone, "The Reasoning Behind the Architecture"]
# ----------------------------------------------------------------------------

def words_for(q_len: int) -> int:
    """Number of 64-bit words per node mask (two words for up to 128 nodes)."""
    return (q_len + 63) // 64


def check_parents(parents: np.ndarray) -> None:
    """Raise ValueError unless ``parents`` is a topologically ordered tree."""
    parents = np.asarray(parents)
    if parents.ndim != 1 or parents.size == 0:
        raise ValueError("parents must be a non-empty 1-D array")
    if int(parents[0]) != -1:
        raise ValueError("parent[0] must be -1 (node 0 is the verified token)")
    for i in range(1, parents.size):
        p = int(parents[i])
        if not (0 <= p < i):
            raise ValueError(f"parent[{i}] = {p} is not an earlier node")


def ancestor_masks(parents: np.ndarray) -> list[int]:
    """Ancestor-or-self sets as Python ints, built in node order:
    mask(0) = bit 0;  mask(i) = mask(parent(i)) | bit(i)."""
    check_parents(parents)
    masks: list[int] = []
    for i, p in enumerate(np.asarray(parents).tolist()):
        own = 1 << i
        masks.append(own if p < 0 else (masks[p] | own))
    return masks


def pack_mask(mask: int, n_words: int) -> np.ndarray:
    """Split an integer bitmask into 64-bit words, least significant first."""
    out = np.zeros(n_words, dtype=np.uint64)
    for w in range(n_words):
        out[w] = np.uint64((mask >> (64 * w)) & 0xFFFFFFFFFFFFFFFF)
    return out


def build_visibility(parents: np.ndarray):
    """parents int [B, q] -> (vis uint64 [B, q, W], depth int32 [B, q]).

    Bit j of row i (word j // 64, bit j % 64) is set iff node j is an
    ancestor of node i or node i itself; depth(i) = |ancestors-or-self| - 1.
    """
    parents = np.asarray(parents)
    B, q = parents.shape
    W = words_for(q)
    vis = np.zeros((B, q, W), dtype=np.uint64)
    depth = np.zeros((B, q), dtype=np.int32)
    for b in range(B):
        masks = ancestor_masks(parents[b])
        for i, m in enumerate(masks):
            vis[b, i] = pack_mask(m, W)
            depth[b, i] = bin(m).count("1") - 1
    return vis, depth


def unpack_row(vis_row: np.ndarray, q_len: int) -> np.ndarray:
    """Boolean visibility of the q_len tree keys for one query node."""
    bits = np.zeros(q_len, dtype=bool)
    for j in range(q_len):
        bits[j] = (int(vis_row[j // 64]) >> (j % 64)) & 1
    return bits


# ----------------------------------------------------------------------------
# Verify attention  [Checkpoint, "The Message"; Final, "Input Knowledge Required"]
# ----------------------------------------------------------------------------

def key_mask(prefix_len: int, vis_row: np.ndarray, q_len: int) -> np.ndarray:
    """[ones over the prefix | tree visibility] for one query node."""
    return np.concatenate([np.ones(prefix_len, dtype=bool), unpack_row(vis_row, q_len)])


def _attend(q_lat_row, q_pe_row, c_kv, k_pe, mask, scale):
    """One query row against keys 0..N-1 (N = len(mask)); float64 throughout.
    Returns (o[R], lse)."""
    s = scale * (c_kv @ q_lat_row + k_pe @ q_pe_row)
    s = np.where(mask, s, -np.inf)
    m = np.max(s)
    e = np.exp(s - m)                      # exactly 0 where masked
    z = np.sum(e)
    lse = m + math.log(z)
    o = (e / z) @ c_kv
    return o, lse


def verify_attn(q_lat, q_pe, c_kv, k_pe, prefix_lens, vis, scale):
    """Tree-verify attention, float64.

    q_lat [B, q, H, R], q_pe [B, q, H, P], c_kv [B, S, R], k_pe [B, S, P]
    (the tree's own latents already appended at rows L_b .. L_b+q-1),
    prefix_lens [B], vis uint64 [B, q, W].
    Returns o [B, q, H, R] and lse [B, q, H] (natural log, scale included).

    One sequence at a time: scores for all (token, head) rows against keys
    0 .. L_b+q-1 in one matrix product, the mask applied per token, then a
    row-wise log-sum-exp and a weighted sum of the c_kv rows.
    """
    q_lat = np.asarray(q_lat, dtype=np.float64)
    q_pe = np.asarray(q_pe, dtype=np.float64)
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_pe = np.asarray(k_pe, dtype=np.float64)
    B, q, H, R = q_lat.shape
    o = np.zeros((B, q, H, R), dtype=np.float64)
    lse = np.zeros((B, q, H), dtype=np.float64)
    for b in range(B):
        L = int(prefix_lens[b])
        N = L + q
        if N > c_kv.shape[1]:
            raise ValueError("prefix_len + q_len exceeds the cache capacity")
        keys_lat = c_kv[b, :N]                          # [N, R]
        keys_pe = k_pe[b, :N]                           # [N, P]
        for t in range(q):
            mask = key_mask(L, vis[b, t], q)            # [N]
            s = scale * (q_lat[b, t] @ keys_lat.T + q_pe[b, t] @ keys_pe.T)   # [H, N]
            s = np.where(mask[None, :], s, -np.inf)
            m = np.max(s, axis=1, keepdims=True)
            e = np.exp(s - m)
            z = np.sum(e, axis=1, keepdims=True)
            lse[b, t] = (m + np.log(z))[:, 0]
            o[b, t] = (e / z) @ keys_lat
    return o, lse


def verify_attn_rows(q_lat, q_pe, c_kv, k_pe, prefix_lens, vis, scale, rows):
    """The same definition for a list of (b, t, h) rows only (used where the
    full output is too large to compute on the CPU).  Inputs may be float64
    arrays or callables returning float64 rows; returns (o [n, R], lse [n])."""
    out_o, out_lse = [], []
    q = vis.shape[1]
    for (b, t, h) in rows:
        L = int(prefix_lens[b])
        N = L + q
        mask = key_mask(L, vis[b, t], q)
        o, l = _attend(np.asarray(q_lat[b, t, h], np.float64), np.asarray(q_pe[b, t, h], np.float64),
                       np.asarray(c_kv[b, :N], np.float64), np.asarray(k_pe[b, :N], np.float64),
                       mask, scale)
        out_o.append(o)
        out_lse.append(l)
    return np.stack(out_o), np.asarray(out_lse)


# ----------------------------------------------------------------------------
# Split-prefix partials and their merge (log-sum-exp identity)
# ----------------------------------------------------------------------------

def attend_chunk(q_lat_row, q_pe_row, c_kv, k_pe, mask, scale):
    """Attention restricted to one chunk of keys: (normalised o, lse); an
    empty or fully masked chunk gives (zeros, -inf)."""
    if not np.any(mask):
        return np.zeros(c_kv.shape[1], dtype=np.float64), -np.inf
    return _attend(q_lat_row, q_pe_row, c_kv, k_pe, mask, scale)


def merge_partials(o_parts, lse_parts):
    """Combine per-chunk results over the chunk axis (axis 0).

    lse = ln sum_k exp(lse_k);  o = sum_k exp(lse_k - lse) * o_k,
    where each o_k is the chunk's normalised output.  Chunks with
    lse_k = -inf carry no weight.  A row whose chunks are all empty gets
    lse = -inf and o = 0.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = np.max(lse_parts, axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - m_safe[None]), 0.0)
    z = np.sum(w, axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, z, 1.0)), -np.inf)
    zz = np.where(finite, z, 1.0)
    o = np.sum(w[..., None] * o_parts, axis=0) / zz[..., None]
    return o, lse


# ----------------------------------------------------------------------------
# Accepted-path gather  [Checkpoint, "The Message": post-verify compaction]
# ----------------------------------------------------------------------------

def gather_accepted(cache, prefix_lens, accepted, n_accepted):
    """Return a copy of ``cache`` [B, S, C] in which, for every sequence b and
    k < n_accepted[b], row L_b + k holds what row L_b + accepted[b, k] held
    before the call.  All other rows are unchanged."""
    old = np.array(cache, copy=True)
    new = np.array(cache, copy=True)
    B = old.shape[0]
    for b in range(B):
        L = int(prefix_lens[b])
        for k in range(int(n_accepted[b])):
            new[b, L + k] = old[b, L + int(accepted[b, k])]
    return new


# ----------------------------------------------------------------------------
# Greedy tree accept  [Checkpoint, "The Message": tree_accept, greedy-exact;
# Milestone, "Mistakes and Incorrect Assumptions": walks bounded]
# ----------------------------------------------------------------------------

def tree_accept(parents, tokens, target_pred):
    """Greedy acceptance of a verified draft tree, one sequence at a time.

    parents     int [B, q], parent[0] = -1, 0 <= parent[i] < i
    tokens      int [B, q], the draft token of each node (node 0: the
                verified token)
    target_pred int [B, q], the target model's greedy next token after each
                node (argmax of its logits at that node)

    Returns (accepted [B, q] int32 node indices, -1 past the end,
    n_accepted [B] int32, bonus [B] int32): starting at the root, repeatedly
    move to the lowest-index child c of the current node u whose token equals
    target_pred[u]; stop when no child matches.  accepted lists the visited
    nodes from the root; bonus = target_pred[last accepted node].
    """
    parents = np.asarray(parents)
    tokens = np.asarray(tokens)
    target_pred = np.asarray(target_pred)
    B, q = parents.shape
    for b in range(B):
        check_parents(parents[b])
    accepted = np.full((B, q), -1, dtype=np.int32)
    n_acc = np.zeros(B, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    for b in range(B):
        u = 0
        path = [0]
        for _ in range(q):                      # a path has at most q nodes
            want = target_pred[b, u]
            nxt = None
            for c in range(1, q):               # children in index order
                if parents[b, c] == u and tokens[b, c] == want:
                    nxt = c
                    break
            if nxt is None:
                break
            u = nxt
            path.append(u)
        accepted[b, :len(path)] = path
        n_acc[b] = len(path)
        bonus[b] = target_pred[b, u]
    return accepted, n_acc, bonus


# ----------------------------------------------------------------------------
# Best-first tree build  [Milestone, "The Context: Why This Commit Exists",
# "The Reasoning Behind the Architecture"; Final, "Input Knowledge Required"]
# ----------------------------------------------------------------------------

def build_tree(topk_tokens, topk_logprobs, root_tokens, q):
    """Best-first draft tree from per-position top-k candidates.

    topk_tokens   int [B, D, K]    K best draft tokens of each draft position
    topk_logprobs float [B, D, K]  their log-probabilities, best first
    root_tokens   int [B]          the verified token (node 0)
    q             nodes per tree (budget), 1 <= q

    Returns a dict of arrays (int32 unless noted):
      parents [B, q], tokens [B, q], depth [B, q], logw float64 [B, q],
      first_child [B, q], next_sibling [B, q] (-1: none), n_nodes [B]
    Nodes past n_nodes are padding (parent 0, token -1, depth 1, logw -inf,
    no links).
    """
    import heapq
    topk_tokens = np.asarray(topk_tokens)
    lp = np.asarray(topk_logprobs)
    B, D, K = topk_tokens.shape
    out = {
        "parents": np.zeros((B, q), np.int32), "tokens": np.full((B, q), -1, np.int32),
        "depth": np.ones((B, q), np.int32), "logw": np.full((B, q), -np.inf),
        "first_child": np.full((B, q), -1, np.int32), "next_sibling": np.full((B, q), -1, np.int32),
        "n_nodes": np.zeros(B, np.int32),
    }
    for b in range(B):
        parents = [-1]
        depth = [0]
        logw = [0.0]
        tokens = [int(root_tokens[b])]
        last_child = {}
        heap = []            # (-logw, push order, depth, rank, parent node)
        order = 0

        def push_children(node):
            """A created node puts all K of its children on the heap, best rank first."""
            nonlocal order
            d = depth[node] + 1
            if d > D:
                return
            for j in range(K):
                heapq.heappush(heap, (-(logw[node] + float(lp[b, d - 1, j])), order, d, j, node))
                order += 1

        push_children(0)
        while len(parents) < q and heap:
            negw, _, d, j, par = heapq.heappop(heap)
            node = len(parents)
            parents.append(par)
            depth.append(d)
            logw.append(-negw)
            tokens.append(int(topk_tokens[b, d - 1, j]))
            if par in last_child:
                out["next_sibling"][b, last_child[par]] = node
            else:
                out["first_child"][b, par] = node
            last_child[par] = node
            push_children(node)
        n = len(parents)
        out["n_nodes"][b] = n
        out["parents"][b, :n] = parents
        out["parents"][b, 0] = -1
        out["tokens"][b, :n] = tokens
        out["depth"][b, :n] = depth
        out["depth"][b, 0] = 0
        out["logw"][b, :n] = logw
    return out


# ----------------------------------------------------------------------------
# Around the verify: split_q + absorb_qk + RoPE, cache append, absorb_vc
# [Checkpoint, "The Message"; Final, "Input Knowledge Required"]
# ----------------------------------------------------------------------------

def rope_neox(x, pos, theta):
    """NeoX rotary embedding of x [..., P] at integer positions pos [...]:
    the pair (x[i], x[i + P/2]) turns by pos * theta^(-2i/P)."""
    x = np.asarray(x, dtype=np.float64)
    P = x.shape[-1]
    half = P // 2
    inv = np.asarray(theta, dtype=np.float64) ** (-(2.0 * np.arange(half)) / P)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def tree_positions(prefix_lens, depth):
    """Position of tree node t of sequence b: L_b + depth(t)."""
    return np.asarray(prefix_lens, np.int64)[:, None] + np.asarray(depth, np.int64)


def absorb_q(q, w_kc_t, prefix_lens, depth, dn, theta):
    """q [B, T, H, dn + P] -> (q_lat [B, T, H, R], q_pe [B, T, H, P]):
    q_lat[b, t, h, r] = sum_i q[b, t, h, i] * w_kc_t[h, r, i] (i < dn) and
    q_pe = rope(q[..., dn:], L_b + depth[b, t])."""
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w_kc_t, dtype=np.float64)
    q_nope, q_rope = q[..., :dn], q[..., dn:]
    q_lat = np.einsum("bthi,hri->bthr", q_nope, w)
    pos = tree_positions(prefix_lens, depth)
    q_pe = rope_neox(q_rope, pos[:, :, None], theta)
    return q_lat, q_pe


def absorb_o(o_lat, w_vc):
    """o_lat [B, T, H, R] -> o [B, T, H, dv]: o[b, t, h, j] = sum_r w_vc[h, j, r] o_lat[b, t, h, r]."""
    return np.einsum("bthr,hjr->bthj", np.asarray(o_lat, np.float64), np.asarray(w_vc, np.float64))


def append_tree_kv(cache, c_kv_new, k_rope_new, prefix_lens, depth, theta):
    """Cache append of the tree tokens: row L_b + t of sequence b gets the
    token's latent c_kv_new[b, t] and its rotary key rotated at L_b +
    depth[b, t].  cache [B, S, R + P] (returned as a new float64 array)."""
    new = np.array(cache, dtype=np.float64, copy=True)
    c = np.asarray(c_kv_new, np.float64)
    k = np.asarray(k_rope_new, np.float64)
    R = c.shape[-1]
    pos = tree_positions(prefix_lens, depth)
    kr = rope_neox(k, pos, theta)
    for b in range(new.shape[0]):
        L = int(prefix_lens[b])
        T = c.shape[1]
        new[b, L:L + T, :R] = c[b]
        new[b, L:L + T, R:] = kr[b]
    return new
