// Best-first draft tree from the drafter's per-position top-k candidates.
//
// "The Milestone Commit: Cementing a Native DDTree Inference Engine", sections
// "The Context: Why This Commit Exists" (the tree was built on the host with a
// heap, a device-host round trip per decode step that a device kernel removes)
// and "The Reasoning Behind the Architecture" (one work unit per request,
// double-precision logw accumulation, first-child / next-sibling links sorted
// by log-probability); "The Final Commit: Cementing a Native DDTree Inference
// Engine for Kimi K2.6", section "Input Knowledge Required" (best-first from
// top-k logits).
//
// Reading used (the pages give no listing): the drafter supplies, for draft
// position d = 1..D, its K best tokens with log-probabilities sorted best
// first; every node at depth d - 1 has those K tokens as candidate children.
// The root (the verified token) has logw 0; a child of rank j has
// logw = logw(parent) + logprob[d][j], in double precision.  Nodes are created
// in order of decreasing logw until the budget of q nodes is reached or no
// candidate remains; candidates are offered lazily (a created node offers its
// parent's next-ranked child, then its own best child), and equal logw goes to
// the candidate offered first.  Leftover budget slots are padding: children
// of the root with token -1, depth 1, logw -inf.
//
// gfx950 mapping: one wave64 per request.  The live candidates (at most q)
// sit in registers, two slots per lane; each creation step is one wave-wide
// arg-max over (logw, offer order), then at most two new candidates are
// written into slots.  The log-probabilities a build can touch (the first
// min(D, q - 1) positions, the first min(K, q) ranks) are staged in LDS
// first; tokens, links and depths are written after the loop from LDS.
#include "kdt_common.hpp"

namespace kdt {

constexpr int kTreeMaxK = 64;                   // ranks per position the build can use
constexpr int kTreeLpMax = (KDT_MAX_Q_LEN - 1) * kTreeMaxK;   // staged log-probabilities

struct Cand {
  double w;      // logw of the candidate node (-inf: empty slot)
  double base;   // logw of its parent
  int order;     // offer order (ties: smaller wins); INT_MAX when empty
  int d, j, par; // depth, rank, parent node
};

__device__ __forceinline__ bool better(double wa, int oa, double wb, int ob) {
  return wa > wb || (wa == wb && oa < ob);
}

__device__ __forceinline__ double shfl_xor_d(double x, int m) {
  const unsigned long long u = __double_as_longlong(x);
  const int lo = __shfl_xor((int)(u & 0xffffffffull), m);
  const int hi = __shfl_xor((int)(u >> 32), m);
  return __longlong_as_double(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

__global__ __launch_bounds__(64) void build_tree_kernel(
    const int32_t* __restrict__ topk_tokens, const float* __restrict__ topk_logprobs,
    const int32_t* __restrict__ root_tokens, int D, int K, int q, int32_t* __restrict__ parents,
    int32_t* __restrict__ tokens, int32_t* __restrict__ depth, double* __restrict__ logw,
    int32_t* __restrict__ first_child, int32_t* __restrict__ next_sibling, int32_t* __restrict__ n_nodes) {
  __shared__ float s_lp[kTreeLpMax];
  __shared__ int s_par[KDT_MAX_Q_LEN], s_dep[KDT_MAX_Q_LEN], s_rank[KDT_MAX_Q_LEN];
  __shared__ int s_first[KDT_MAX_Q_LEN], s_next[KDT_MAX_Q_LEN], s_last[KDT_MAX_Q_LEN];
  __shared__ double s_w[KDT_MAX_Q_LEN];

  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int Du = min(D, q - 1);                 // positions a build of q nodes can reach
  const int Ku = min(K, q);                     // ranks it can reach
  const float* lp = topk_logprobs + (int64_t)b * D * K;
  for (int i = lane; i < Du * Ku; i += 64) s_lp[i] = lp[(int64_t)(i / Ku) * K + i % Ku];
  for (int i = lane; i < KDT_MAX_Q_LEN; i += 64) {
    s_first[i] = -1;
    s_next[i] = -1;
    s_last[i] = -1;
  }
  __syncthreads();

  // two candidate slots per lane: slot s lives in lane s % 64, register s / 64
  Cand c[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) c[k] = Cand{-INFINITY, 0.0, INT_MAX, 0, 0, 0};
  int n = 1;                                    // nodes created (the root)
  int next_order = 0, next_slot = 0;
  if (lane == 0) {
    s_par[0] = -1;
    s_dep[0] = 0;
    s_rank[0] = 0;
    s_w[0] = 0.0;
  }
  if (Du >= 1) {                                // the root's best child
    if (lane == 0) c[0] = Cand{0.0 + (double)s_lp[0], 0.0, 0, 1, 0, 0};
    next_order = 1;
    next_slot = 1;
  }
#pragma unroll 1
  while (n < q) {
    // arg-max over the live candidates: the lane's better slot, then the wave
    const bool pick1 = better(c[1].w, c[1].order, c[0].w, c[0].order);
    double bw = pick1 ? c[1].w : c[0].w;
    int bo = pick1 ? c[1].order : c[0].order;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const double ow = shfl_xor_d(bw, m);
      const int oo = __shfl_xor(bo, m);
      if (better(ow, oo, bw, bo)) {
        bw = ow;
        bo = oo;
      }
    }
    if (bo == INT_MAX) break;                   // no candidate left
    // the owner of the winning slot (offer orders are unique)
    const bool own0 = c[0].order == bo, own1 = c[1].order == bo;
    const unsigned long long ownmask = __ballot(own0 || own1);
    const int owner = __builtin_ctzll(ownmask);
    const int oslot = __shfl((int)own1, owner);
    const Cand win = oslot ? c[1] : c[0];
    const int d = __shfl(win.d, owner), j = __shfl(win.j, owner), par = __shfl(win.par, owner);
    const double base = __shfl(win.base, owner);
    const double w = bw;

    const int node = n++;
    if (lane == 0) {
      s_par[node] = par;
      s_dep[node] = d;
      s_rank[node] = j;
      s_w[node] = w;
      const int last = s_last[par];
      if (last < 0) s_first[par] = node;
      else s_next[last] = node;
      s_last[par] = node;
    }
    // offers: the next-ranked sibling (into the winning slot), then the
    // node's own best child (into a fresh slot)
    Cand sib{-INFINITY, 0.0, INT_MAX, 0, 0, 0};
    if (j + 1 < K && j + 1 < Ku) sib = Cand{base + (double)s_lp[(d - 1) * Ku + j + 1], base, next_order++, d, j + 1, par};
    if (lane == owner) {
      if (oslot) c[1] = sib;
      else c[0] = sib;
    }
    if (d < Du) {
      const Cand ch{w + (double)s_lp[d * Ku], w, next_order++, d + 1, 0, node};
      const int s = next_slot++;
      if (lane == (s & 63)) {
        if (s >> 6) c[1] = ch;
        else c[0] = ch;
      }
    }
  }
  __syncthreads();

  // outputs: created nodes from LDS, padding after them
  for (int i = lane; i < q; i += 64) {
    const int64_t o = (int64_t)b * q + i;
    if (i < n) {
      const int d = s_dep[i];
      parents[o] = s_par[i];
      depth[o] = d;
      tokens[o] = i == 0 ? root_tokens[b] : topk_tokens[((int64_t)b * D + (d - 1)) * K + s_rank[i]];
      if (logw) logw[o] = s_w[i];
      if (first_child) first_child[o] = s_first[i];
      if (next_sibling) next_sibling[o] = s_next[i];
    } else {
      parents[o] = 0;
      depth[o] = 1;
      tokens[o] = -1;
      if (logw) logw[o] = -INFINITY;
      if (first_child) first_child[o] = -1;
      if (next_sibling) next_sibling[o] = -1;
    }
  }
  if (lane == 0 && n_nodes) n_nodes[b] = n;
}

}  // namespace kdt

extern "C" int kdt_build_tree(const int32_t* topk_tokens, const float* topk_logprobs, const int32_t* root_tokens,
                              int32_t B, int32_t D, int32_t K, int32_t q_len, int32_t* parents, int32_t* tokens,
                              int32_t* depth, double* logw, int32_t* first_child, int32_t* next_sibling,
                              int32_t* n_nodes, void* stream) {
  if (!topk_tokens || !topk_logprobs || !root_tokens || !parents || !tokens || !depth) return KDT_ERR_INVALID_ARG;
  if (B <= 0 || D <= 0 || K <= 0 || q_len <= 0) return KDT_ERR_INVALID_ARG;
  if ((int64_t)D * K > 0x7FFFFFFF / 2) return KDT_ERR_UNSUPPORTED;
  if (q_len > KDT_MAX_Q_LEN || (K > kdt::kTreeMaxK && q_len > kdt::kTreeMaxK)) return KDT_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(kdt::build_tree_kernel, dim3(B), dim3(64), 0, static_cast<hipStream_t>(stream), topk_tokens,
                     topk_logprobs, root_tokens, (int)D, (int)K, (int)q_len, parents, tokens, depth, logw,
                     first_child, next_sibling, n_nodes);
  return kdt::launch_status();
}
