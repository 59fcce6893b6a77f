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

}  // namespace kdt
