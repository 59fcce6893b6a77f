// Common device/host helpers for the kdt HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kdt.h"

namespace kdt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;      // MI355X: 8 XCDs, workgroups dispatched round-robin over them

// Workgroup i is dispatched to XCD (i % 8).  Return a logical index such that
// the workgroups placed on one XCD receive a contiguous block of logical
// indices, so neighbouring logical work (same keys, different rows) shares
// that XCD's L2.
__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int per = n / kNumXcd, extra = n % kNumXcd;
  const int x = i % kNumXcd, slot = i / kNumXcd;
  return x * per + (x < extra ? x : extra) + slot;
}

__device__ __forceinline__ void flag_seq(int32_t* seq_status, int b, int32_t flag) {
  if (seq_status) atomicOr(seq_status + b, flag);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? KDT_OK : KDT_ERR_LAUNCH;
}

// Ancestor-or-self bitmasks of a tree of q <= 128 nodes in one wave64 by
// pointer doubling ("The Milestone Commit: Cementing a Native DDTree
// Inference Engine", "The Reasoning Behind the Architecture": a node's mask is
// its parent's mask plus its own bit, two 64-bit words per node).  Lane i owns
// nodes i and i + 64; par[k] is the parent of node lane + 64 k (any value for
// nodes >= q).  After round r every node holds the union of itself and its
// ancestors fewer than 2^r levels up and a pointer 2^r levels up (or -1 past
// the root); seven rounds cover any depth below 128.  The exchange goes
// through this wave's own LDS area s_m (2 words per node) and s_j (one pointer
// per node), updated in place: the wave's LDS instructions execute in order,
// and a node that reads an ancestor already advanced in the same round only
// advances further (every mask stays the union of the ancestors closer than
// its pointer), so no second buffer or barrier is needed.  A parent that is
// not an earlier node (or a root with a parent) counts as none, so no walk can
// cycle or leave the tree; the return value says whether any lane saw one.
__device__ __forceinline__ bool wave_ancestor_masks(const int par[2], int q, uint64_t* s_m, int* s_j, int lane,
                                                    uint64_t m0[2], uint64_t m1[2]) {
  bool bad = false;
  int jmp[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = lane + 64 * k;
    int p = -1;
    m0[k] = 0;
    m1[k] = 0;
    if (i < q) {
      p = par[k];
      const bool ok = (i == 0) ? (p == -1) : (p >= 0 && p < i);
      if (!ok) {
        bad = true;
        p = -1;
      }
      if (i < 64) m0[k] = 1ull << i;
      else m1[k] = 1ull << (i - 64);
    }
    jmp[k] = p;
    s_m[2 * i] = m0[k];
    s_m[2 * i + 1] = m1[k];
    s_j[i] = p;
  }
  // Rounds stop once every pointer has passed the root (a tree of depth d
  // needs ceil(log2(d + 1)) of them); nodes 64.. exist only when q > 64.
  const int nk = q > 64 ? 2 : 1;
#pragma unroll 1
  for (int round = 0; round < 7; ++round) {
    if (!__any((jmp[0] >= 0) | ((nk > 1) & (jmp[1] >= 0)))) break;
    uint64_t a0[2], a1[2];
    int aj[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (k >= nk) break;
      const int j = jmp[k] >= 0 ? jmp[k] : 0;
      a0[k] = s_m[2 * j];
      a1[k] = s_m[2 * j + 1];
      aj[k] = s_j[j];
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (k >= nk) break;
      const int i = lane + 64 * k;
      if (jmp[k] >= 0) {
        m0[k] |= a0[k];
        m1[k] |= a1[k];
        jmp[k] = aj[k];
      }
      s_m[2 * i] = m0[k];
      s_m[2 * i + 1] = m1[k];
      s_j[i] = jmp[k];
    }
  }
  return bad;
}

}  // namespace kdt
