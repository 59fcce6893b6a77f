"""Seeded synthetic inputs for tree-verify MLA-absorb attention.

This module only draws random inputs; it holds none of the attention, mask,
merge or gather arithmetic.  Both the CPU oracle (through the tests) and the
HIP path consume exactly the arrays produced here, so the two sides always see
identical bits.

Workload shapes follow the pages' test configurations:
  * "max budget q_len=65", "batch-64" and "deep-15" tree shapes, from
    "The Milestone Commit: Cementing a Native DDTree Inference Engine",
    sections "The Context: Why This Commit Exists" and "What the Message
    Actually Does";
  * the tiny model's 4 heads and kv_lora_rank 64, from "The Final Commit:
    Cementing a Native DDTree Inference Engine for Kimi K2.6", section
    "The Message" (tiny vs tiny2 configs);
  * kv_lora_rank 512 / rope dim 64 for the K2.6-sized configs.
No public dataset is involved: the pages validate verify attention on random
MLA-shaped tensors ("The Milestone Commit", section "The Thinking Process
Visible in the Reasoning"), and these generators stand in for that.

Conventions
-----------
* Generator: ``numpy.random.Generator(PCG64(seed))``, seed = 20261200 + the
  config's 1-based index.  Draw order: parents, prefix_lens, q_lat, q_pe,
  cache, accepted-node choice.
* Values are drawn as float32 N(0, 1) (queries optionally scaled), then rounded
  to bfloat16 with round-to-nearest-even for the bf16 configs.  bf16 arrays are
  returned as their raw uint16 bit patterns.
* The latent cache is one array ``cache[B, S_cap, R + P]``: columns ``0..R-1``
  hold c_kv, columns ``R..R+P-1`` hold k_pe.  S_cap = max_b(L_b + q) rounded
  up to a multiple of 64.  Tree node t of sequence b sits at row L_b + t.
* Trees are parent arrays in node order: parent[0] = -1 and
  0 <= parent[i] < i (topological, best-first pop order).
"""
from __future__ import annotations

import heapq
import math
from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 20261200


@dataclass(frozen=True)
class Config:
    name: str
    index: int            # 1-based; seed = SEED_BASE + index
    dtype: str            # "f32" or "bf16"
    B: int
    H: int
    R: int                # kv_lora_rank
    P: int                # rope dim
    q_len: int
    prefix: tuple         # ("fixed", L) or ("uniform", lo, hi) inclusive
    tree: str             # "uniform", "best_first", "deep_chain"
    q_scale: float = 1.0  # queries multiplied by this before rounding
    max_acc: int = 0      # accepted-path rows per sequence for the gather (0: path length bound q)
    note: str = ""

    @property
    def D(self) -> int:
        return self.R + self.P

    @property
    def softmax_scale(self) -> float:
        # 1/sqrt(R+P): the tiny configuration states 1/sqrt(80) for R=64, P=16;
        # the same rule is used for every configuration.
        return 1.0 / math.sqrt(self.R + self.P)


CONFIGS = {
    "tiny_fp32": Config("tiny_fp32", 1, "f32", B=1, H=4, R=64, P=16, q_len=9,
                        prefix=("fixed", 32), tree="uniform",
                        note="batch 1, heads 4, R 64, P 16, prefix 32, q_len 9"),
    "max_budget": Config("max_budget", 2, "bf16", B=1, H=16, R=512, P=64, q_len=65,
                         prefix=("fixed", 4096), tree="best_first",
                         note="batch 1, heads 16, prefix 4096, q_len 65 best-first tree"),
    "batched": Config("batched", 3, "bf16", B=64, H=16, R=512, P=64, q_len=17,
                      prefix=("fixed", 2048), tree="uniform",
                      note="batch 64, heads 16, prefix 2048, q_len 17"),
    "long_ctx": Config("long_ctx", 4, "bf16", B=4, H=64, R=512, P=64, q_len=65,
                       prefix=("fixed", 32768), tree="best_first", q_scale=0.5,
                       note="batch 4, heads 64, prefix 32768, q_len 65, q scaled 0.5"),
    "ragged_deep": Config("ragged_deep", 5, "bf16", B=16, H=16, R=512, P=64, q_len=33,
                          prefix=("uniform", 1024, 16384), tree="deep_chain", max_acc=16,
                          note="batch 16, heads 16, prefix U[1024,16384], q_len 33 depth-15 trees"),
}


def config_variant(cfg: Config, **changes) -> Config:
    """A copy of ``cfg`` with some fields replaced (e.g. q_len=1 for the AR case)."""
    d = {k: getattr(cfg, k) for k in cfg.__dataclass_fields__}
    d.update(changes)
    return Config(**d)


# ----------------------------------------------------------------------------
# bf16 bit handling (input preparation only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the uint16 bit patterns.  Inputs here are finite normal draws.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 values of bfloat16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a generated tensor (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# Tree shapes
# ----------------------------------------------------------------------------

def tree_uniform(rng: np.random.Generator, q: int) -> np.ndarray:
    """parent[i] ~ U{0, ..., i-1}."""
    p = np.empty(q, dtype=np.int32)
    p[0] = -1
    for i in range(1, q):
        p[i] = rng.integers(0, i)
    return p


def tree_chain(q: int) -> np.ndarray:
    p = np.arange(-1, q - 1, dtype=np.int32)
    return p


def tree_star(q: int) -> np.ndarray:
    p = np.zeros(q, dtype=np.int32)
    p[0] = -1
    return p


def _node_depths(parents: np.ndarray) -> np.ndarray:
    d = np.zeros(len(parents), dtype=np.int64)
    for i in range(1, len(parents)):
        d[i] = d[parents[i]] + 1
    return d


def tree_best_first(rng: np.random.Generator, q: int, max_branch: int = 4,
                    max_depth: int = 8) -> np.ndarray:
    """A best-first-shaped draft tree (this generator's own definition).

    Each expanded node draws k ~ U{1..max_branch} candidate children whose
    log-probabilities are the logs of a Dirichlet(1,...,1) draw sorted in
    descending order.  A max-heap on the cumulative float64 log-weight pops
    candidates; each pop becomes the next node index and is expanded in turn.
    Candidates deeper than ``max_depth`` are never pushed; ties go to the
    earlier-created candidate.  If the heap empties before q nodes exist, the
    whole draw is repeated with the same generator.
    """
    while True:
        parents = [-1]
        depths = [0]
        heap: list = []
        counter = 0

        def expand(node: int, logw: float):
            nonlocal counter
            k = int(rng.integers(1, max_branch + 1))
            probs = np.sort(rng.dirichlet(np.ones(k)))[::-1]
            for pr in probs:
                if depths[node] + 1 > max_depth:
                    continue
                lw = logw + math.log(max(float(pr), 1e-300))
                heapq.heappush(heap, (-lw, counter, node))
                counter += 1

        expand(0, 0.0)
        while len(parents) < q and heap:
            neg_lw, _, par = heapq.heappop(heap)
            idx = len(parents)
            parents.append(par)
            depths.append(depths[par] + 1)
            expand(idx, -neg_lw)
        if len(parents) == q:
            return np.asarray(parents, dtype=np.int32)


def tree_deep_chain(rng: np.random.Generator, q: int, chain: int = 16,
                    side_max_depth: int = 14) -> np.ndarray:
    """Nodes 0..chain-1 form a chain (depth chain-1); every later node i picks
    parent ~ U{0..i-1}, redrawn until the new node's depth is <= side_max_depth."""
    p = np.empty(q, dtype=np.int32)
    p[0] = -1
    depth = np.zeros(q, dtype=np.int64)
    for i in range(1, min(chain, q)):
        p[i] = i - 1
        depth[i] = i
    for i in range(chain, q):
        while True:
            c = int(rng.integers(0, i))
            if depth[c] + 1 <= side_max_depth:
                break
        p[i] = c
        depth[i] = depth[c] + 1
    return p


def path_to(parents: np.ndarray, node: int) -> np.ndarray:
    """Root-to-node index list (the accepted path that ends at ``node``)."""
    out = []
    c = int(node)
    while c >= 0:
        out.append(c)
        c = int(parents[c])
    return np.asarray(out[::-1], dtype=np.int32)


# ----------------------------------------------------------------------------
# Full inputs
# ----------------------------------------------------------------------------

@dataclass
class Inputs:
    cfg: Config
    parents: np.ndarray        # int32 [B, q]
    prefix_lens: np.ndarray    # int32 [B]
    q_lat: np.ndarray          # [B, q, H, R]  uint16 bf16 bits or float32
    q_pe: np.ndarray           # [B, q, H, P]
    cache: np.ndarray          # [B, S_cap, R+P]
    accepted: np.ndarray       # int32 [B, max_acc]  (rows beyond n_accepted are 0)
    n_accepted: np.ndarray     # int32 [B]
    extra: dict = field(default_factory=dict)

    @property
    def S_cap(self) -> int:
        return self.cache.shape[1]

    def f64(self, name: str) -> np.ndarray:
        return to_f64(getattr(self, name), self.cfg.dtype)


def _values(rng: np.random.Generator, shape, dtype: str, scale: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x = (x * np.float32(scale)).astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


def make_tree(rng: np.random.Generator, kind: str, q: int) -> np.ndarray:
    if q == 1:
        return np.array([-1], dtype=np.int32)
    if kind == "uniform":
        return tree_uniform(rng, q)
    if kind == "best_first":
        return tree_best_first(rng, q)
    if kind == "deep_chain":
        return tree_deep_chain(rng, q)
    if kind == "chain":
        return tree_chain(q)
    if kind == "star":
        return tree_star(q)
    raise ValueError(f"unknown tree kind {kind!r}")


def generate(cfg: Config, seed: int | None = None, *, prefix_override=None,
             cap_round: int = 64) -> Inputs:
    """Draw every input of one verify + gather call for ``cfg``."""
    rng = np.random.Generator(np.random.PCG64(SEED_BASE + cfg.index if seed is None else seed))
    B, q, H, R, P = cfg.B, cfg.q_len, cfg.H, cfg.R, cfg.P
    parents = np.stack([make_tree(rng, cfg.tree, q) for _ in range(B)]).astype(np.int32)
    if prefix_override is not None:
        prefix_lens = np.asarray(prefix_override, dtype=np.int32).reshape(B)
    elif cfg.prefix[0] == "fixed":
        prefix_lens = np.full(B, cfg.prefix[1], dtype=np.int32)
    else:
        lo, hi = cfg.prefix[1], cfg.prefix[2]
        prefix_lens = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    q_lat = _values(rng, (B, q, H, R), cfg.dtype, cfg.q_scale)
    q_pe = _values(rng, (B, q, H, P), cfg.dtype, cfg.q_scale)
    need = int(prefix_lens.max()) + q
    S_cap = max(cap_round, -(-need // cap_round) * cap_round)
    cache = _values(rng, (B, S_cap, R + P), cfg.dtype)
    max_acc = cfg.max_acc if cfg.max_acc > 0 else q
    accepted = np.zeros((B, max_acc), dtype=np.int32)
    n_acc = np.zeros(B, dtype=np.int32)
    for b in range(B):
        if cfg.tree == "deep_chain" and b == 0 and q >= 16:
            node = 15                                   # the full depth-15 chain
        else:
            node = int(rng.integers(0, q))
        path = path_to(parents[b], node)[:max_acc]
        accepted[b, :len(path)] = path
        n_acc[b] = len(path)
    return Inputs(cfg, parents, prefix_lens, q_lat, q_pe, cache, accepted, n_acc)


def rng_for(tag: int) -> np.random.Generator:
    """A generator for ad-hoc test inputs, seeded off the same base."""
    return np.random.Generator(np.random.PCG64(SEED_BASE + 1000 + int(tag)))


def accept_inputs(parents: np.ndarray, seed: int, vocab: int = 32, p_follow: float = 0.75):
    """Draft tokens and target predictions for a batch of trees (random draws
    only).  Siblings carry distinct tokens (as a top-k expansion gives); the
    target's prediction at a node is, with probability p_follow, the token of
    one of its children (chosen uniformly), and otherwise a token none of its
    children carries.  Node 0's token is the verified token.

    Returns (tokens [B, q], target_pred [B, q]) as int32."""
    rng = np.random.Generator(np.random.PCG64(SEED_BASE + 2000 + int(seed)))
    parents = np.asarray(parents)
    B, q = parents.shape
    tokens = np.zeros((B, q), dtype=np.int32)
    pred = np.zeros((B, q), dtype=np.int32)
    for b in range(B):
        children = [[] for _ in range(q)]
        for i in range(1, q):
            children[int(parents[b, i])].append(i)
        tokens[b, 0] = rng.integers(vocab)
        for u in range(q):
            kids = children[u]
            if kids:
                # a node with more children than the vocabulary has letters
                # draws from a vocabulary just large enough
                tokens[b, kids] = rng.choice(max(vocab, len(kids) + 1), size=len(kids), replace=False)
        for u in range(q):
            kids = children[u]
            taken = set(int(tokens[b, c]) for c in kids)
            if kids and rng.random() < p_follow:
                pred[b, u] = tokens[b, kids[int(rng.integers(len(kids)))]]
            else:
                free = [v for v in range(max(vocab, len(kids) + 1)) if v not in taken]
                pred[b, u] = free[int(rng.integers(len(free)))]
    return tokens, pred


def tree_topk_inputs(B: int, D: int, K: int, seed: int, vocab: int = 1000, temp: float = 1.0):
    """Drafter output for the best-first tree build (random draws only): for
    each of B requests and D draft positions, the K most likely tokens of a
    softmax over `vocab` random logits (N(0, 1) / temp), with their float32
    log-probabilities sorted best first, plus a verified root token.

    Returns (topk_tokens int32 [B, D, K], topk_logprobs float32 [B, D, K],
    root_tokens int32 [B])."""
    rng = np.random.Generator(np.random.PCG64(SEED_BASE + 3000 + int(seed)))
    logits = rng.standard_normal((B, D, vocab)) / temp
    logits -= logits.max(axis=-1, keepdims=True)
    logp = logits - np.log(np.exp(logits).sum(axis=-1, keepdims=True))
    order = np.argsort(-logp, axis=-1, kind="stable")[..., :K]
    tokens = order.astype(np.int32)
    lps = np.take_along_axis(logp, order, axis=-1).astype(np.float32)
    roots = rng.integers(0, vocab, size=B).astype(np.int32)
    return tokens, lps, roots


def absorb_inputs(B: int, T: int, H: int, dn: int, P: int, R: int, dv: int, seed: int):
    """Inputs of the steps around the verify (random draws only), all bf16 bit
    patterns: the per-head query projection q [B, T, H, dn + P] (N(0, 1)),
    the absorbed key weights w_kc_t [H, R, dn] (N(0, 1/dn)), the value
    weights w_vc [H, dv, R] (N(0, 1/R)), a latent attention output
    o_lat [B, T, H, R], and the tree tokens' new latents c_kv_new [B, T, R]
    and rotary keys k_rope_new [B, T, P] (N(0, 1))."""
    rng = np.random.Generator(np.random.PCG64(SEED_BASE + 4000 + int(seed)))
    f = lambda shape, sd: f32_to_bf16_bits((rng.standard_normal(shape) * sd).astype(np.float32))
    return {
        "q": f((B, T, H, dn + P), 1.0),
        "w_kc_t": f((H, R, dn), dn ** -0.5),
        "w_vc": f((H, dv, R), R ** -0.5),
        "o_lat": f((B, T, H, R), 1.0),
        "c_kv_new": f((B, T, R), 1.0),
        "k_rope_new": f((B, T, P), 1.0),
    }
