// Ancestor-or-self visibility bitmasks from parent pointers.
//
// "The Milestone Commit: Cementing a Native DDTree Inference Engine", section
// "The Reasoning Behind the Architecture": a node's mask is its parent's mask
// with its own bit added, two 64-bit words per node cover up to 65 nodes, and
// the sequential O(n) build is followed by a parallel O(n^2) expansion.
//
// On gfx950 the sequential chain is replaced by pointer doubling inside one
// wavefront (wave_ancestor_masks): the wave owns one sequence, lane i owns tree
// nodes i and i + 64, and seven rounds of one LDS exchange each cover any tree
// of at most 128 nodes regardless of its depth.  The packed rows are written
// directly (they are the rows of the full q x q matrix).  The verify kernel
// runs the same function when it is handed parents instead of masks.
//
// Safety bound ("The Milestone Commit", section "Mistakes and Incorrect
// Assumptions", the tree_accept crash on cyclic random trees): a parent that is
// not an earlier node is treated as "no parent", so no walk can cycle or leave
// the tree; the sequence is flagged KDT_SEQ_BAD_TREE.
#include "kdt_common.hpp"

namespace kdt {

__global__ __launch_bounds__(64) void build_visibility_kernel(
    const int32_t* __restrict__ parents, int q, uint64_t* __restrict__ vis,
    int32_t* __restrict__ depth, int32_t* __restrict__ seq_status) {
  __shared__ uint64_t s_m[2 * KDT_MAX_Q_LEN];
  __shared__ int s_j[KDT_MAX_Q_LEN];

  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int W = (q + 63) >> 6;
  const int32_t* par = parents + (int64_t)b * q;
  int p[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) p[k] = lane + 64 * k < q ? par[lane + 64 * k] : -1;
  uint64_t m0[2], m1[2];      // masks of node lane (index 0) and lane + 64 (index 1)
  const bool bad = wave_ancestor_masks(p, q, s_m, s_j, lane, m0, m1);

#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = lane + 64 * k;
    if (i < q) {
      uint64_t* row = vis + ((int64_t)b * q + i) * W;
      row[0] = m0[k];
      if (W > 1) row[1] = m1[k];
      if (depth) depth[(int64_t)b * q + i] = __popcll(m0[k]) + __popcll(m1[k]) - 1;
    }
  }
  // any lane that saw an invalid parent flags the sequence
  if (__any(bad) && lane == 0) flag_seq(seq_status, b, KDT_SEQ_BAD_TREE);
}

}  // namespace kdt

extern "C" int kdt_build_visibility(const int32_t* parents, int32_t B, int32_t q_len,
                                    uint64_t* vis, int32_t* depth, int32_t* seq_status,
                                    void* stream) {
  if (!parents || !vis) return KDT_ERR_INVALID_ARG;
  if (B <= 0 || q_len <= 0) return KDT_ERR_INVALID_ARG;
  if (q_len > KDT_MAX_Q_LEN) return KDT_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(kdt::build_visibility_kernel, dim3(B), dim3(64), 0,
                     static_cast<hipStream_t>(stream), parents, (int)q_len, vis, depth, seq_status);
  return kdt::launch_status();
}
