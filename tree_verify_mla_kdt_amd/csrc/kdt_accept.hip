// Greedy acceptance of a verified draft tree.
//
// "The Checkpoint: Committing a Working Native DDTree Engine", section "The
// Message": the decode loop runs tree build -> verify -> tree accept -> cache
// compaction, and greedy tree decoding must reproduce greedy autoregressive
// decoding token for token.  Starting at the root (the verified token), the
// accepted path moves to a child whose draft token equals the target's greedy
// prediction at the current node, as long as one exists; the prediction at
// the last accepted node is the bonus token.  When several children carry the
// predicted token the lowest-index one (the earliest in best-first order) is
// taken.  Walks are bounded by the tree size: "The Milestone Commit:
// Cementing a Native DDTree Inference Engine", section "Mistakes and
// Incorrect Assumptions" (the accept crash on cyclic random trees).
//
// One wavefront per sequence; lane i owns nodes i and i + 64.  Each step of
// the walk is one ballot over "my parent is the current node and my token is
// its prediction": the lowest set bit is the next node.  The prediction of
// the current node comes from the lane that owns it (a uniform readlane), so
// the walk touches memory only to load the tree and to write the result.
#include "kdt_common.hpp"

namespace kdt {

__global__ __launch_bounds__(64) void tree_accept_kernel(
    const int32_t* __restrict__ parents, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ target_pred, int q, int32_t* __restrict__ accepted,
    int32_t* __restrict__ n_accepted, int32_t* __restrict__ bonus, int32_t* __restrict__ seq_status) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t base = (int64_t)b * q;

  // nodes lane (index 0) and lane + 64 (index 1); absent nodes get parent -2,
  // which no current node matches
  int par[2], tok[2], prd[2];
  bool bad = false;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = lane + 64 * k;
    par[k] = -2;
    tok[k] = 0;
    prd[k] = 0;
    if (i < q) {
      int p = parents[base + i];
      const bool ok = (i == 0) ? (p == -1) : (p >= 0 && p < i);
      if (!ok) {
        bad = true;
        p = -2;               // a node with an invalid parent cannot be reached
      }
      par[k] = (i == 0) ? -2 : p;
      tok[k] = tokens[base + i];
      prd[k] = target_pred[base + i];
    }
  }
  if (__any(bad) && lane == 0) flag_seq(seq_status, b, KDT_SEQ_BAD_TREE);

  // The walk.  acc[k] of lane j holds accepted[j + 64 k].
  int acc[2] = {-1, -1};
  if (lane == 0) acc[0] = 0;
  int u = 0, n = 1;
#pragma unroll 1
  for (int step = 1; step < q; ++step) {
    const int want = u < 64 ? __builtin_amdgcn_readlane(prd[0], u) : __builtin_amdgcn_readlane(prd[1], u - 64);
    const uint64_t m0 = __ballot(par[0] == u && tok[0] == want);
    const uint64_t m1 = __ballot(par[1] == u && tok[1] == want);
    if (m0 == 0 && m1 == 0) break;
    u = m0 ? __builtin_ctzll(m0) : 64 + __builtin_ctzll(m1);
    if (lane == n) acc[0] = u;
    if (lane + 64 == n) acc[1] = u;
    ++n;
  }
  const int last = u < 64 ? __builtin_amdgcn_readlane(prd[0], u) : __builtin_amdgcn_readlane(prd[1], u - 64);

#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = lane + 64 * k;
    if (i < q) accepted[base + i] = acc[k];
  }
  if (lane == 0) {
    n_accepted[b] = n;
    if (bonus) bonus[b] = last;
  }
}

}  // namespace kdt

extern "C" int kdt_tree_accept(const int32_t* parents, const int32_t* tokens, const int32_t* target_pred,
                               int32_t B, int32_t q_len, int32_t* accepted, int32_t* n_accepted,
                               int32_t* bonus, int32_t* seq_status, void* stream) {
  if (!parents || !tokens || !target_pred || !accepted || !n_accepted) return KDT_ERR_INVALID_ARG;
  if (B <= 0 || q_len <= 0) return KDT_ERR_INVALID_ARG;
  if (q_len > KDT_MAX_Q_LEN) return KDT_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(kdt::tree_accept_kernel, dim3(B), dim3(64), 0, static_cast<hipStream_t>(stream), parents,
                     tokens, target_pred, (int)q_len, accepted, n_accepted, bonus, seq_status);
  return kdt::launch_status();
}
