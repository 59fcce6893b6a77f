// Post-accept compaction: gather the accepted path's latents into the rows
// right after the prefix.
//
// "The Checkpoint: Committing a Working Native DDTree Engine", section "The
// Message": the engine keeps a KV cache with "cache append + post-verify
// compaction" and, after acceptance, gathers the accepted-path latents.
//
// Layout of the work: one workgroup per (layer, sequence, column slice).  The
// slice is 16 vector lanes wide (16 x 16 B = 256 B of each row for 16-byte
// vectors); the workgroup's 256 threads cover up to 16 rows of the slice per
// pass, and every accepted row of the slice is first read into registers, then
// the workgroup synchronises, then all rows are written.  Column slices are
// disjoint, so "read everything before writing anything" holds per slice and
// overlapping source/destination rows (e.g. accepted = [0, 2, 3]) are safe.
// Consecutive threads touch consecutive 16-byte vectors of one row, so reads
// and writes are coalesced.
#include "kdt_common.hpp"

namespace kdt {

constexpr int kGatherThreads = 256;
constexpr int kSliceVecs = 16;                       // vectors per row slice
constexpr int kRowsPerPass = kGatherThreads / kSliceVecs;   // 16
constexpr int kMaxRowsPerThread = KDT_MAX_Q_LEN / kRowsPerPass;  // 8

template <typename V>
__global__ __launch_bounds__(kGatherThreads) void gather_accepted_kernel(
    char* __restrict__ cache, int64_t cache_sb, int64_t cache_ss, int64_t capacity,
    int64_t layer_stride, int B, int q, int row_vecs, int slices,
    const int32_t* __restrict__ prefix_lens, const int32_t* __restrict__ accepted,
    const int32_t* __restrict__ n_accepted, int max_acc,
    int32_t* __restrict__ new_prefix_lens, int32_t* __restrict__ seq_status) {
  // strides arrive in bytes
  // blockIdx.x enumerates (layer, sequence, slice) with the slice fastest
  const int64_t wg = blockIdx.x;
  const int slice = (int)(wg % slices);
  const int b = (int)((wg / slices) % B);
  const int layer = (int)(wg / ((int64_t)slices * B));
  const int tid = threadIdx.x;
  const int vec = slice * kSliceVecs + (tid % kSliceVecs);
  const int r0 = tid / kSliceVecs;

  const int32_t* acc = accepted + (int64_t)b * max_acc;
  const int n_max = max_acc < q ? max_acc : q;
  // The accepted indices are requested together with the prefix length and
  // the path length (every entry below max_acc is inside the caller's array),
  // so the source rows are one memory round trip away instead of two.
  int src_of[kMaxRowsPerThread];
#pragma unroll
  for (int k = 0; k < kMaxRowsPerThread; ++k) {
    const int row = r0 + k * kRowsPerPass;
    src_of[k] = row < n_max ? acc[row] : -1;
  }
  const int L = prefix_lens[b];
  int n = n_accepted[b];
  const bool first = (layer == 0 && slice == 0 && tid == 0);
  if (L < 0 || (int64_t)L + q > capacity) {
    if (first) flag_seq(seq_status, b, KDT_SEQ_BAD_LEN);
    return;
  }
  if (n < 0 || n > n_max) {
    if (first) flag_seq(seq_status, b, KDT_SEQ_BAD_INDEX);
    n = n < 0 ? 0 : n_max;
  }
  if (first && new_prefix_lens) new_prefix_lens[b] = L + n;

  char* base = cache + layer * layer_stride + b * cache_sb + (int64_t)L * cache_ss;

  V buf[kMaxRowsPerThread];
  bool take[kMaxRowsPerThread];
  bool bad_index = false;
#pragma unroll
  for (int k = 0; k < kMaxRowsPerThread; ++k) {
    const int row = r0 + k * kRowsPerPass;
    take[k] = false;
    if (row < n && vec < row_vecs) {
      const int src = src_of[k];
      if (src >= 0 && src < q) {
        buf[k] = *reinterpret_cast<const V*>(base + (int64_t)src * cache_ss + (int64_t)vec * sizeof(V));
        take[k] = true;
      } else {
        bad_index = true;
      }
    }
  }
  __syncthreads();   // every source row of this slice is in registers
#pragma unroll
  for (int k = 0; k < kMaxRowsPerThread; ++k) {
    const int row = r0 + k * kRowsPerPass;
    if (take[k])
      *reinterpret_cast<V*>(base + (int64_t)row * cache_ss + (int64_t)vec * sizeof(V)) = buf[k];
  }
  if (bad_index && layer == 0 && slice == 0) flag_seq(seq_status, b, KDT_SEQ_BAD_INDEX);
}

template <typename V>
static int launch_gather(char* cache, int64_t sb, int64_t ss, int64_t capacity, int64_t ls,
                         int B, int q, int row_bytes, int layers, const int32_t* pl,
                         const int32_t* acc, const int32_t* nacc, int max_acc, int32_t* npl,
                         int32_t* st, hipStream_t stream) {
  const int row_vecs = row_bytes / (int)sizeof(V);
  const int slices = (row_vecs + kSliceVecs - 1) / kSliceVecs;
  const int64_t grid = (int64_t)slices * B * layers;
  if (grid > 0x7FFFFFFF) return KDT_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(gather_accepted_kernel<V>, dim3((unsigned)grid), dim3(kGatherThreads), 0,
                     stream, cache, sb, ss, capacity, ls, B, q, row_vecs, slices, pl, acc, nacc,
                     max_acc, npl, st);
  return launch_status();
}

}  // namespace kdt

extern "C" int kdt_gather_accepted(int32_t dtype, int32_t B, int32_t q_len, int32_t row_elems,
                                   void* cache, int64_t cache_sb, int64_t cache_ss,
                                   int64_t capacity, int32_t num_layers, int64_t layer_stride,
                                   const int32_t* prefix_lens, const int32_t* accepted,
                                   const int32_t* n_accepted, int32_t max_acc,
                                   int32_t* new_prefix_lens, int32_t* seq_status, void* stream) {
  if (!cache || !prefix_lens || !accepted || !n_accepted) return KDT_ERR_INVALID_ARG;
  if (B <= 0 || q_len <= 0 || row_elems <= 0 || num_layers <= 0 || capacity < q_len)
    return KDT_ERR_INVALID_ARG;
  if (max_acc <= 0 || max_acc > q_len) return KDT_ERR_INVALID_ARG;
  if (cache_ss < row_elems || cache_sb < 0 || layer_stride < 0) return KDT_ERR_INVALID_ARG;
  if (new_prefix_lens && new_prefix_lens == prefix_lens) return KDT_ERR_INVALID_ARG;
  if (q_len > KDT_MAX_Q_LEN) return KDT_ERR_UNSUPPORTED;
  int esz;
  if (dtype == KDT_F32) esz = 4;
  else if (dtype == KDT_BF16) esz = 2;
  else return KDT_ERR_UNSUPPORTED;

  const int64_t row_bytes = (int64_t)row_elems * esz;
  const int64_t sb = cache_sb * esz, ss = cache_ss * esz, ls = layer_stride * esz;
  if (row_bytes > (int64_t)1 << 30) return KDT_ERR_UNSUPPORTED;
  // widest vector that divides the row, the strides and the base address
  const uintptr_t a = reinterpret_cast<uintptr_t>(cache) | (uintptr_t)row_bytes | (uintptr_t)sb |
                      (uintptr_t)ss | (uintptr_t)ls;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* c = static_cast<char*>(cache);
  if ((a & 15) == 0)
    return kdt::launch_gather<uint4>(c, sb, ss, capacity, ls, B, q_len, (int)row_bytes, num_layers,
                                     prefix_lens, accepted, n_accepted, max_acc, new_prefix_lens,
                                     seq_status, s);
  if ((a & 7) == 0)
    return kdt::launch_gather<uint2>(c, sb, ss, capacity, ls, B, q_len, (int)row_bytes, num_layers,
                                     prefix_lens, accepted, n_accepted, max_acc, new_prefix_lens,
                                     seq_status, s);
  if ((a & 3) == 0)
    return kdt::launch_gather<uint32_t>(c, sb, ss, capacity, ls, B, q_len, (int)row_bytes,
                                        num_layers, prefix_lens, accepted, n_accepted, max_acc,
                                        new_prefix_lens, seq_status, s);
  return kdt::launch_gather<uint16_t>(c, sb, ss, capacity, ls, B, q_len, (int)row_bytes, num_layers,
                                      prefix_lens, accepted, n_accepted, max_acc, new_prefix_lens,
                                      seq_status, s);
}
