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
// candidate remains: a plain heap onto which each created node pushes all K
// of its children, equal logw going to the child of the earlier created
// parent, then to the lower rank (the heap's push order).  Leftover budget
// slots are padding: children of the root with token -1, depth 1, logw -inf.
//
// Lazy offers: with the log-probabilities sorted best first, a node's
// children leave that heap in rank order, so only each parent's best
// remaining child can be the next node.  The kernel therefore holds just
// those: a created node offers its own best child, and a candidate, once
// created, offers its next-ranked sibling.  Ties are keyed on (parent index,
// rank), the push order of the full heap, so both create the same nodes in
// the same order, ties included.
//
// gfx950 mapping: one wave64 per request.  The live candidates are kept
// sorted best first across the lanes, one per lane, so the best candidate is
// always in lane 0.  A creation step reads lane 0, forms the (at most two)
// new offers, counts with two ballots how many remaining candidates beat each
// offer, and rebuilds the sorted list in one pass: every lane takes its own
// candidate, its neighbour's from one lane up or one lane down (whole-wave DPP
// shifts, plain VALU moves), or one of the offers.  Sixty-four lanes are
// enough for q <= 128: at most n live candidates exist after n nodes, and only
// the best q - n of them can still be created, so a candidate pushed past lane
// 63 (possible only once n > 64) could never have been chosen.  Each
// candidate carries the log-probabilities of its own next sibling and first
// child, read from LDS when it is offered, so a step waits on no memory.  The
// log-probabilities a build can touch (the first min(D, q - 1) positions, the
// first min(K, q) ranks) are staged in LDS first; parents, depths, ranks and
// logw are kept in LDS and written out after the loop, and the sibling links
// are derived there from the parents in creation order.
#include "kdt_common.hpp"

namespace kdt {

constexpr int kTreeMaxK = 64;                   // ranks per position the build can use
constexpr int kTreeLpMax = (KDT_MAX_Q_LEN - 1) * kTreeMaxK;   // staged log-probabilities

// One candidate: logw, its parent's logw, tie key parent * kTreeMaxK + rank
// (smaller wins; INT_MAX marks an empty lane), depth | rank << 8 | parent << 16,
// and the log-probabilities of its next sibling and of its first child.
struct Cand {
  double w, base;
  int order, pk;
  float lsib, lch;
};

// (evaluated without short-circuit, so it compiles to compares and masks)
__device__ __forceinline__ bool better(double wa, int oa, double wb, int ob) {
  return (wa > wb) | ((wa == wb) & (oa < ob));
}

// Whole-wave lane shifts (DPP): lane i receives lane i + 1's value (UP) or
// lane i - 1's (DOWN).  The lane with no source (63 for UP, 0 for DOWN)
// receives zero; the rebuild below never selects that value (lane i takes
// the UP value only while i < p1 <= 63, and lane 0 never takes DOWN).
constexpr int kDppWaveShl1 = 0x130;
constexpr int kDppWaveShr1 = 0x138;
template <int CTRL>
__device__ __forceinline__ int shift_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, true);
}
template <int CTRL>
__device__ __forceinline__ float shift_f(float x) {
  return __int_as_float(shift_i<CTRL>(__float_as_int(x)));
}
template <int CTRL>
__device__ __forceinline__ double shift_d(double x) {
  const unsigned long long u = __double_as_longlong(x);
  const int lo = shift_i<CTRL>((int)(u & 0xffffffffull));
  const int hi = shift_i<CTRL>((int)(u >> 32));
  return __longlong_as_double(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}
template <int CTRL>
__device__ __forceinline__ Cand shift_c(const Cand& c) {
  return Cand{shift_d<CTRL>(c.w), shift_d<CTRL>(c.base), shift_i<CTRL>(c.order), shift_i<CTRL>(c.pk),
              shift_f<CTRL>(c.lsib), shift_f<CTRL>(c.lch)};
}

__device__ __forceinline__ double lane0_d(double x) {
  const unsigned long long u = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_readlane((int)(u & 0xffffffffull), 0);
  const int hi = __builtin_amdgcn_readlane((int)(u >> 32), 0);
  return __longlong_as_double(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ float lane0_f(float x) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)); }

__global__ __launch_bounds__(64) void build_tree_kernel(
    const int32_t* __restrict__ topk_tokens, const float* __restrict__ topk_logprobs,
    const int32_t* __restrict__ root_tokens, int D, int K, int q, int32_t* __restrict__ parents,
    int32_t* __restrict__ tokens, int32_t* __restrict__ depth, double* __restrict__ logw,
    int32_t* __restrict__ first_child, int32_t* __restrict__ next_sibling, int32_t* __restrict__ n_nodes) {
  __shared__ float s_lp[kTreeLpMax];
  __shared__ int s_par[KDT_MAX_Q_LEN], s_dep[KDT_MAX_Q_LEN], s_rank[KDT_MAX_Q_LEN];
  __shared__ double s_w[KDT_MAX_Q_LEN];

  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int Du = min(D, q - 1);                 // positions a build of q nodes can reach
  const int Ku = min(K, q);                     // ranks it can reach
  const float* lp = topk_logprobs + (int64_t)b * D * K;
  for (int i = lane; i < Du * Ku; i += 64) s_lp[i] = lp[(int64_t)(i / Ku) * K + i % Ku];
  if (lane == 0) {
    s_par[0] = -1;
    s_dep[0] = 0;
    s_rank[0] = 0;
    s_w[0] = 0.0;
  }
  __syncthreads();

  // the sorted frontier: lane i holds the i-th best live candidate
  Cand c{-INFINITY, 0.0, INT_MAX, 0, 0.0f, 0.0f};
  int n = 1;                                    // nodes created (the root)
  if (Du >= 1) {                                // the root's best child
    if (lane == 0) c = Cand{0.0 + (double)s_lp[0], 0.0, 0, 1, Ku > 1 ? s_lp[1] : 0.0f, Du > 1 ? s_lp[Ku] : 0.0f};
  }
#pragma unroll 1
  while (n < q) {
    const int o0 = __builtin_amdgcn_readlane(c.order, 0);
    if (o0 == INT_MAX) break;                   // no candidate left
    const double w = lane0_d(c.w), base = lane0_d(c.base);
    const int pk = __builtin_amdgcn_readlane(c.pk, 0);
    const float lsib = lane0_f(c.lsib), lch = lane0_f(c.lch);
    const int d = pk & 0xff, j = (pk >> 8) & 0xff, par = pk >> 16;
    const int node = n++;
    if (lane == 0) {
      s_par[node] = par;
      s_dep[node] = d;
      s_rank[node] = j;
      s_w[node] = w;
    }
    // offers: the next-ranked sibling, then the node's own best child (an
    // absent offer is an empty candidate); the log-probabilities they carry
    // are read at clamped indices and selected
    const bool has_s = j + 1 < Ku, has_c = d < Du;
    const float l_s2 = s_lp[j + 2 < Ku ? (d - 1) * Ku + j + 2 : 0];
    const float l_c1 = s_lp[has_c && Ku > 1 ? d * Ku + 1 : 0];
    const float l_c0 = s_lp[d + 1 < Du ? (d + 1) * Ku : 0];
    const Cand sib{has_s ? base + (double)lsib : -INFINITY, base, has_s ? par * kTreeMaxK + j + 1 : INT_MAX,
                   d | (j + 1) << 8 | par << 16, j + 2 < Ku ? l_s2 : 0.0f, lch};
    const Cand ch{has_c ? w + (double)lch : -INFINITY, w, has_c ? node * kTreeMaxK : INT_MAX, (d + 1) | node << 16,
                  Ku > 1 ? l_c1 : 0.0f, d + 1 < Du ? l_c0 : 0.0f};
    const bool sib_first = better(sib.w, sib.order, ch.w, ch.order);
    const double hi_w = sib_first ? sib.w : ch.w, lo_w = sib_first ? ch.w : sib.w;
    const double hi_b = sib_first ? sib.base : ch.base, lo_b = sib_first ? ch.base : sib.base;
    const int hi_o = sib_first ? sib.order : ch.order, lo_o = sib_first ? ch.order : sib.order;
    const int hi_p = sib_first ? sib.pk : ch.pk, lo_p = sib_first ? ch.pk : sib.pk;
    const float hi_s = sib_first ? sib.lsib : ch.lsib, lo_s = sib_first ? ch.lsib : sib.lsib;
    const float hi_c = sib_first ? sib.lch : ch.lch, lo_c = sib_first ? ch.lch : sib.lch;
    // after removing lane 0, the list is lanes 1..63; hi goes to position p1,
    // lo to p2 (the lists are sorted, so each ballot is a run from lane 1)
    const bool beats_hi = (lane >= 1) & better(c.w, c.order, hi_w, hi_o);
    const bool beats_lo = (lane >= 1) & better(c.w, c.order, lo_w, lo_o);
    const int p1 = __builtin_popcountll(__ballot(beats_hi));
    const int p2 = __builtin_popcountll(__ballot(beats_lo)) + 1;
    const Cand up = shift_c<kDppWaveShl1>(c), down = shift_c<kDppWaveShr1>(c);
    // lane < p1: up; p1: hi; p1 < lane < p2: its own (one place further from
    // the front); p2: lo; beyond: down
    const bool t_up = lane < p1, t_hi = lane == p1, t_own = lane < p2, t_lo = lane == p2;
#define KDT_PICK(f, hv, lv) (t_up ? up.f : t_hi ? (hv) : t_own ? c.f : t_lo ? (lv) : down.f)
    c = Cand{KDT_PICK(w, hi_w, lo_w), KDT_PICK(base, hi_b, lo_b), KDT_PICK(order, hi_o, lo_o),
             KDT_PICK(pk, hi_p, lo_p), KDT_PICK(lsib, hi_s, lo_s), KDT_PICK(lch, hi_c, lo_c)};
#undef KDT_PICK
  }
  __syncthreads();

  // sibling links in creation order: first_child[p] is the first node created
  // with parent p, next_sibling[i] the next node after i with i's parent
  int fc[2] = {-1, -1}, nsib[2] = {-1, -1}, mypar[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) mypar[r] = lane + 64 * r < n ? s_par[lane + 64 * r] : -2;
#pragma unroll 1
  for (int k = n - 1; k >= 1; --k) {
    const int pk = s_par[k];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = lane + 64 * r;
      if (pk == i) fc[r] = k;
      if (k > i && pk == mypar[r]) nsib[r] = k;
    }
  }

  // outputs: created nodes from LDS, padding after them
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = lane + 64 * r;
    if (i >= q) break;
    const int64_t o = (int64_t)b * q + i;
    if (i < n) {
      const int d = s_dep[i];
      parents[o] = s_par[i];
      depth[o] = d;
      tokens[o] = i == 0 ? root_tokens[b] : topk_tokens[((int64_t)b * D + (d - 1)) * K + s_rank[i]];
      if (logw) logw[o] = s_w[i];
      if (first_child) first_child[o] = fc[r];
      if (next_sibling) next_sibling[o] = nsib[r];
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
