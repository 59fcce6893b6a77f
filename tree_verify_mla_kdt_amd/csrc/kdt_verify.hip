// Tree-verify MLA-absorb attention: split-prefix verify kernel + cross-split
// log-sum-exp merge, for gfx950 (CDNA4, wave64, MFMA).
//
// What is computed ("The Checkpoint: Committing a Working Native DDTree
// Engine", section "The Message", KV-cache scheme; "The Final Commit:
// Cementing a Native DDTree Inference Engine for Kimi K2.6", section "Input
// Knowledge Required", absorbed MLA): the q_len tree tokens of a sequence,
// each with H heads, attend over the cached latent rows [prefix | tree] under
// the mask [ones | ancestor-or-self visibility].  Score of key j for row
// (t, h): scale * (q_lat . c_kv[j] + q_pe . k_pe[j]); output: softmax-weighted
// sum of c_kv rows, plus the row's log-sum-exp.
//
// Design (gfx950-first; the pages give no kernel design for this step):
// * The latent cache is shared by every head, so for one sequence the
//   (token, head) rows form the M dimension of two dense contractions:
//   S^T = K * Q^T over D = R + P, and O^T = V^T * P^T over keys (V = c_kv).
//   Both run on v_mfma_f32_32x32x16_bf16 (bf16) or v_mfma_f32_32x32x2_f32
//   (fp32).
// * A workgroup is 4 waves (one per SIMD) and owns a tile of rows of one
//   sequence and one split of its key range, in one of four layouts:
//   1: 128 rows, each wave 32 rows and all R output columns (its latent Q
//      fragments in registers for the whole key loop, its rope fragments
//      read from LDS every tile, its 32 x R fp32 accumulators in the
//      accumulation registers);
//   2: 64 rows, each pair of waves shares 32 rows, computes the same scores
//      and splits the output columns (half the value work per wave, a
//      deeper tile ring);
//   3: as 2, but the pair splits the score contraction by depth and adds the
//      partner's partial scores through LDS;
//   4: 64 rows as two row blocks x two key streams: each wave owns all R
//      columns of its 32 rows (registers as in layout 1) and takes every
//      other key tile (no contraction step repeated, each tile read by two
//      waves); the two streams are combined through LDS after the last tile.
// * Keys stream through LDS in tiles of 32 rows x (R + P); all four waves read
//   the same tile, so each K/V byte crosses L2 -> LDS once per workgroup.
// * Computing S^T (keys along the MFMA rows) leaves every lane holding 16
//   scores of ONE query row.  The row max needs one cross-half exchange, the
//   running sum needs none until the end, and the softmax weights are already
//   laid out as the B operand of the value contraction: no shuffles.
// * Online softmax in the log2 domain against a per-row reference max fixed at
//   the first visible key.  Weights stay below 2^32 for any realistic score
//   range, so the accumulators are never rescaled (a rescale would need a
//   read-modify-write of every accumulation register every tile).  A row whose
//   max outgrows its reference by more than that makes its wave redo the
//   split once against the exact max, which it has tracked meanwhile.
// * K/V tiles rotate through three (layouts 1, 3) or four (layouts 2, 4) LDS
//   buffers and are copied straight from HBM into LDS with
//   buffer_load_dwordx4 ... lds, so staging costs no registers and all but one
//   buffer are in flight while one tile is computed.  The value operand is
//   read with the gfx950 transposing LDS load (ds_read_b64_tr_b16) from the
//   same key-major tile the score operand uses.
// * Masking costs nothing on prefix tiles; only tiles that reach the tree
//   segment or the end of the split test bits.  The visibility words come from
//   the caller, or, given parent pointers, from a pointer doubling that the
//   workgroups whose split reaches the tree run before their key loop.
// * Split-prefix: a sequence's keys are cut into splits (fixed size, or
//   adaptive: in proportion to the sequence's length); each split writes a
//   normalised partial (bf16 for bf16 inputs, float32 on request, with
//   streaming stores) and its log-sum-exp, and the merge kernel recombines
//   them.  With a single split the verify kernel writes the final output
//   directly.  The balanced schedule instead cuts all sequences' key tiles,
//   laid end to end, into equal ranges, one per gang of workgroups, which
//   walk from one sequence into the next (bal_init / bal_next).
// * Workgroup indices are remapped so the workgroups on one XCD take
//   consecutive work units (all row tiles of one key split, or one gang),
//   which keeps their shared K/V stream in that XCD's L2.
// * The score MFMAs are inline asm with a VGPR destination (see
//   Mfma<__bf16>::mma_acc_v); the build scans the compiled code for the one
//   operand hazard the compiler does not guard there.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>

#include "kdt_common.hpp"

namespace kdt {

constexpr int kBM = 128;          // query rows per workgroup in layout 1 (half in layouts 2, 3)
constexpr int kBN = 32;           // keys per LDS tile
constexpr int kThreads = 256;     // 4 waves
constexpr int kCU = 256;          // MI355X compute units (split heuristic)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRefSlack = 32.0f;   // max weight 2^32 against the reference (log2 units)
// LDS operand fragments kept in flight ahead of the MFMA that consumes them
// (LDS latency under load is a few hundred cycles, one MFMA about forty).
#ifndef KDT_SCORE_PREFETCH
#define KDT_SCORE_PREFETCH 4
#endif
#ifndef KDT_VALUE_PREFETCH
#define KDT_VALUE_PREFETCH 2
#endif

template <typename T>
struct Mfma;

template <>
struct Mfma<__bf16> {
  typedef bf16x8 frag;
  static constexpr int KW = 8;     // operand elements per lane
  static constexpr int KMF = 16;   // contraction depth of one MFMA
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // The score chain's form: the 32x32 tile it accumulates stays in ordinary
  // VGPRs.  (The compiler's own form puts it in accumulation registers, which
  // the output blocks fill, and moves one output block out and back every key
  // tile.)  Written as inline asm, which the compiler's hazard checks do not
  // see, so: the chain accumulates back to back into the same registers, which
  // the hardware allows; the destination never overlaps the A or B operand
  // (early clobber, or tied to C); and score_ready() must separate the last
  // MFMA from the first vector read of the tile.
  __device__ static __forceinline__ f32x16 mma_first_v(frag a, frag b) {
    f32x16 d;
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
    return d;
  }
  __device__ static __forceinline__ void mma_acc_v(frag a, frag b, f32x16& c) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  }
  // 24 wait states: more than a 32x32x16 MFMA's result needs before a vector
  // instruction reads it
  __device__ static __forceinline__ void score_ready(f32x16& c) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c));
  }
  __device__ static __forceinline__ frag pack(const float* p) {
    frag f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = (__bf16)p[j];
    return f;
  }
  __device__ static __forceinline__ frag zero() {
    frag f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = (__bf16)0.0f;
    return f;
  }
};

template <>
struct Mfma<float> {
  typedef float frag;
  static constexpr int KW = 1;
  static constexpr int KMF = 2;
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ frag pack(const float* p) { return p[0]; }
  __device__ static __forceinline__ frag zero() { return 0.0f; }
};

struct VerifyArgs {
  const void* q_lat; int64_t q_lat_sb, q_lat_st, q_lat_sh;
  const void* q_pe;  int64_t q_pe_sb, q_pe_st, q_pe_sh;
  const void* c_kv;  int64_t c_kv_sb, c_kv_ss;
  const void* k_pe;  int64_t k_pe_sb, k_pe_ss;
  int64_t capacity;
  const int32_t* prefix_lens;
  const uint64_t* vis;
  const int32_t* parents;   // masks derived in the kernel from these when vis is null
  void* out; int64_t out_sb, out_st, out_sh;
  float* lse;
  void* part_o;         // float32 or bf16 (part_bf16), tiled
  float* part_lse;
  int32_t* seq_status;
  float scale_log2;
  int B, q, H, M, W, n_rt, n_blk, max_splits, split_keys, max_prefix_len, layout;
  // 0: fixed splits of split_keys keys; > 0: adaptive splits, this being the
  // key tiles of the longest sequence the launch allows (see split_range)
  int tiles_max;
  int group_mul;        // order of the (sequence, split) groups (coprime to B * max_splits)
  int compact;          // number the pieces with work (adaptive splits over several sequences)
  // Work-balanced schedule (gang > 0): gang = row tiles that move through the
  // keys together, n_grp = such groups per sequence, gangs = gangs in the
  // launch (the grid is gangs * gang workgroups)
  int gang, n_grp, gangs;
  int piece_units;      // balanced schedule: units a stream's start-up costs, in key tiles
  int span_keys;        // the most keys of one piece (cache rows one buffer descriptor spans)
  int q_rows_uniform;   // query rows m = t * H + h sit at one byte stride (q_lat and q_pe)
  int part_bf16;        // partial outputs in bf16 (else float32)
  // Merge inside the split kernel (partial mode only): the split workgroups
  // of a row tile meet at a bounded wait on their state word
  // counters[b * n_rt + rt] and share the merge.
  int fuse;
  int32_t* counters;
  int64_t spin_ticks;   // longest wait, in 100 MHz ticks (0: do not wait)
};

// The value of C-layout register v of a 32x32 MFMA result held by a lane in
// half hh (lane / 32) sits in row 8*(v/4) + 4*hh + (v%4) of the 32-row block.
__device__ __forceinline__ int c_row(int v, int hh) { return 8 * (v >> 2) + 4 * hh + (v & 3); }

// Combine a value with the one held by the lane 32 away.  v_permlane32_swap
// (called with the same register twice) returns, in some order, the lane's
// own value and its partner's, so a symmetric operation of the pair is the
// same on both lanes; it is a plain VALU instruction, unlike a DS permute.
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Scheduling fence: MFMAs and LDS accesses keep their program order around it,
// while VALU, SALU and transcendental instructions may still move across.
__device__ __forceinline__ void fence_mem_mfma() { __builtin_amdgcn_sched_barrier(0x0406); }

template <typename T>
__device__ __forceinline__ void store4(T* dst, const float* v);
template <>
__device__ __forceinline__ void store4<float>(float* dst, const float* v) {
  *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
}
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* dst, const float* v) {
  *reinterpret_cast<bf16x4*>(dst) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
}
// Device-coherent 16-byte store and load (cache policy sc1: the access is
// coherent at device scope, across the XCDs' separate L2 caches; the store is
// also streaming, nt).  The split workgroups exchange partials this way inside
// one launch: a writer's stores are complete once its vmcnt reaches zero, and
// a reader's sc1 loads then see them, without the whole-L2 write-back and
// invalidation of a device-scope fence.  base must be wave-uniform.
typedef int i32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}
template <typename V>
__device__ __forceinline__ void store16_coherent(void* base, uint32_t off, V v) {
  static_assert(sizeof(V) == 16, "16-byte store");
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4v, v), coherent_rsrc(base), off, 0, 18);
}
template <typename V>
__device__ __forceinline__ V load16_coherent(const void* base, uint32_t off) {
  static_assert(sizeof(V) == 16, "16-byte load");
  return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(coherent_rsrc(base), off, 0, 16));
}

// LDS image of one key tile.  Two regions: kBN rows of the c_kv part (RC
// 16-byte chunks per row) followed by kBN rows of the k_pe part (PC chunks).
// Chunk c of row k is stored at chunk position c ^ swz_of<NCH>(k).  The LDS
// serves 64 banks x 4 bytes, i.e. one 256-byte window (16 chunks) per cycle:
//  * rows of a multiple of 16 chunks start on the same banks, so the swizzle
//    s16(k) = ((k & 3) << 2) | ((k >> 2) & 3) permutes 16-chunk groups.  It is
//    a bijection on k % 16 (16 consecutive keys reading one chunk for the
//    score operand hit 16 different chunks), and for 4 consecutive keys 4j..4j+3
//    its upper two bits are 0, 1, 2, 3, so a transposing read (4 keys x 4
//    adjacent chunks) covers all 16 chunks of the window;
//  * rows of 8 chunks (128 bytes) pair up in one window; s8(k) = (k >> 1) & 7
//    makes the 16 (key, chunk) reads of 16 consecutive keys distinct.
__device__ __forceinline__ int swz16(int k) { return ((k & 3) << 2) | ((k >> 2) & 3); }
__device__ __forceinline__ int swz8(int k) { return (k >> 1) & 7; }

template <int NCH>
__device__ __forceinline__ int swz_of(int row) {
  if constexpr (NCH % 16 == 0) return swz16(row);
  else if constexpr (NCH % 8 == 0) return swz8(row);
  else return 0;
}

template <int NCH>
__device__ __forceinline__ int region_off(int row, int chunk) {
  return (row * NCH + (chunk ^ swz_of<NCH>(row))) << 4;
}

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

// ds_read_b64_tr_b16: within each 16-lane group, lane j receives element
// (j % 4) of the 8-byte load issued by lane 4e + j / 4, for e = 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (stride 0, num_records in bytes), wave-uniform.
// Loads at or past num_records return zero instead of faulting.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)p),
               __builtin_amdgcn_readfirstlane((int)((uint32_t)(p >> 32) & 0xFFFFu)),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)p);
}

// buffer_load_dwordx4 ... lds: the 16 bytes of lane i land at LDS byte
// address m0 + 16 i.  Issued as inline asm on purpose: the compiler does not
// track these LDS writes, so it neither delays later reads of the other tile
// buffers for them nor drains them at barriers; the kernel orders them itself
// (s_waitcnt vmcnt, then a workgroup barrier, before a tile buffer is read).
// Nothing else in the kernel uses m0.
__device__ __forceinline__ void dma16_to_lds(i32x4 rs, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(rs), "s"(soff)
      : "memory", "m0");
}
// The same with the scalar offset soff_a + soff_b: the add fills the wait
// state the copy needs after the m0 write, in place of the s_nop.
__device__ __forceinline__ void dma16_to_lds2(i32x4 rs, uint32_t lds, uint32_t voff, uint32_t soff_a,
                                              uint32_t soff_b) {
  uint32_t soff;
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_add_u32 %0, %3, %4\n\t"
      "buffer_load_dwordx4 %2, %5, %0 offen lds"
      : "=&s"(soff)
      : "s"(lds), "v"(voff), "s"(soff_a), "s"(soff_b), "s"(rs)
      : "memory", "m0", "scc");
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (N < 64): this wave's older tile copies have
// landed in LDS and its own LDS reads have returned.  The 6-bit vmcnt field
// is split: bits 3:0 of the immediate and bits 15:14.
template <int N>
__device__ __forceinline__ void wait_vmem_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every outstanding load, including tile copies meant to stay in
// flight).  The memory clobber keeps the compiler from moving any access
// across it; the wait above provides the ordering the tile ring needs.
__device__ __forceinline__ void tile_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt lgkmcnt(0) alone: this wave's LDS accesses are done (tile copies
// may stay in flight).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Loads one wave issues for a region of SLOTS 16-byte chunks when wave-loads
// are dealt round-robin to the four waves: the minimum over the waves.
constexpr int min_wave_loads(int slots) { return (slots / 64) / (kThreads / 64); }

// Start the copy of one region of a key tile straight into LDS: every
// buffer_load_dwordx4 ... lds writes 64 consecutive 16-byte LDS slots, one per
// lane, so each lane fetches the global chunk that belongs in its slot.  Rows
// at or past `nrows` (the end of the split) re-read row nrows-1: the softmax
// gives them zero weight, and this keeps every LDS value a finite cache value.
// `wave` must be wave-uniform (an SGPR): the LDS destination and, for regions
// of 64 chunks per row, the source row are then scalar and each load needs a
// single per-lane offset register.
// Wave-loads per wave for a region of ROWS x NCH 16-byte chunks (the maximum
// over the waves; some waves may issue one fewer).
template <int ROWS, int NCH>
constexpr int region_wave_loads() { return (ROWS * NCH / 64 + kThreads / 64 - 1) / (kThreads / 64); }

// The jj-th wave-load of this wave for one region (nothing if this wave has
// fewer).  stage_region issues them all.  The region's first row sits at byte
// base_off of buffer rs, rows ss bytes apart; lds is its LDS byte address.
// FUSED: the offset add inside the copy's asm (fewer instructions where the
// copies share the wave's issue slots with a dependent MFMA chain).
template <int ROWS, int NCH, bool FUSED = false>
__device__ __forceinline__ void stage_one(i32x4 rs, uint32_t base_off, uint32_t ss, int nrows, uint32_t lds, int wave,
                                          int lane, int jj) {
  constexpr int SLOTS = ROWS * NCH;
  static_assert(SLOTS % 64 == 0, "tile region must be whole wave loads");
  constexpr int WAVES = kThreads / 64;
  {
    const int j = wave + jj * WAVES;
    if ((SLOTS / 64) % WAVES != 0 && j >= SLOTS / 64) return;
    if constexpr (NCH == 64) {
      // one row per instruction: the row (and its swizzle) is wave-uniform
      const int row = j;
      const uint32_t voff = (uint32_t)(lane ^ swz_of<NCH>(row)) * 16;
      if constexpr (FUSED) {
        // min(row, nrows - 1) * ss as min(row * ss, (nrows - 1) * ss), the
        // first product fixed per wave and piece
        const uint32_t roff = min((uint32_t)row * ss, (uint32_t)(nrows - 1) * ss);
        dma16_to_lds2(rs, __builtin_amdgcn_readfirstlane(lds + j * 1024), voff,
                      __builtin_amdgcn_readfirstlane(base_off), __builtin_amdgcn_readfirstlane(roff));
      } else {
        const int src_row = row < nrows ? row : nrows - 1;
        dma16_to_lds(rs, __builtin_amdgcn_readfirstlane(lds + j * 1024), voff,
                     __builtin_amdgcn_readfirstlane(base_off + (uint32_t)src_row * ss));
      }
    } else {
      const int slot = j * 64 + lane;
      const int row = slot / NCH, pc = slot - row * NCH;
      const int c = pc ^ swz_of<NCH>(row);
      const int src_row = row < nrows ? row : nrows - 1;
      const uint32_t voff = (uint32_t)src_row * ss + (uint32_t)c * 16;
      dma16_to_lds(rs, __builtin_amdgcn_readfirstlane(lds + j * 1024), voff, __builtin_amdgcn_readfirstlane(base_off));
    }
  }
}

template <int ROWS, int NCH>
__device__ __forceinline__ void stage_region(i32x4 rs, uint32_t base_off, uint32_t ss, int nrows, uint32_t lds,
                                             int wave, int lane) {
#pragma unroll
  for (int jj = 0; jj < region_wave_loads<ROWS, NCH>(); ++jj)
    stage_one<ROWS, NCH>(rs, base_off, ss, nrows, lds, wave, lane, jj);
}

// ---------------------------------------------------------------------------
// Cross-split merge: lse = ln sum_k exp(lse_k), o = sum_k exp(lse_k - lse) o_k.
// Partials are in accumulator order (32-row blocks, see the split kernel's
// epilogue), so one wave handles one (sequence, block, column group) of 8
// float32 or 16 bf16 columns: every lane reads 16 bytes per split and the
// wave's reads are one contiguous 1 KB run.  Splits are consumed sixteen at a
// time with a running maximum, so sixteen loads per lane are in flight (one
// memory round trip for up to sixteen splits).  Splits with lse_k = -inf are
// skipped by selection, never by multiplication: their partial output may
// never have been written.
template <typename PT>
struct PartLoad;
template <>
struct PartLoad<float> {
  static constexpr int NV = 4;                  // values per lane per split
  typedef f32x4 raw;
  __device__ static __forceinline__ float get(const raw& r, int i) { return r[i]; }
};
template <>
struct PartLoad<__bf16> {
  static constexpr int NV = 8;
  typedef bf16x8 raw;
  __device__ static __forceinline__ float get(const raw& r, int i) { return (float)r[i]; }
};

// One merge item: the rows of 32-row block blk of sequence b (m < M) and
// column group cg (8 float32 or 16 bf16 partial columns), over splits
// 0 .. ns - 1.  Without WIDE one wave does the item: every lane reads 16
// bytes per split, the wave's reads of one split one contiguous 1 KB run.
// WIDE: the four waves of the workgroup share the item, wave w loading the
// w-th quarter of the splits at once, and wave 0 combines the four (max, sum,
// columns) states through s_st (4 * (NV + 2) * 64 floats of LDS); every wave
// of the workgroup must then call it with the same item.  Splits at or past
// ns are skipped.  COH: the partials
// were stored by other workgroups of the running launch and are read with
// device-coherent loads.  GATE: a split's partial row is loaded only once its
// log-sum-exp has shown it is not empty (for partial buffers where most of
// the max_splits slots of a row are empty; one more memory round trip).
template <typename T, typename PT, bool WIDE, bool COH, bool GATE = false, int U = 16>
__device__ __forceinline__ void merge_item(const PT* __restrict__ part_o, const float* __restrict__ part_lse,
                                           int max_splits, int ns, int M, int H, int R, int n_blk, int b, int blk,
                                           int cg, T* __restrict__ out, int64_t out_sb, int64_t out_st,
                                           int64_t out_sh, float* __restrict__ lse, float* s_st, int wave,
                                           int lane) {
  // (U: splits loaded in one round trip; fewer for launches with few splits,
  // whose registers then leave room for more waves)
  constexpr int NV = PartLoad<PT>::NV;
  constexpr int CW = 2 * NV;                    // columns per item
  typedef typename PartLoad<PT>::raw raw;
  const int hh = lane >> 5;
  const int m = blk * 32 + (lane & 31);
  const bool row_ok = m < M;
  // (WIDE: the quarters are of max_splits, so the grouping of the sums, and
  // so the result, does not depend on how many splits the sequence uses)
  const int per = WIDE ? (max_splits + 3) / 4 : ns;
  const int kb = WIDE ? wave * per : 0;
  const int ke = row_ok ? min(ns, kb + per) : kb;   // padding rows load nothing
  const float* pl = part_lse + (int64_t)b * max_splits * M + (row_ok ? m : 0);
  const int64_t split_stride = (int64_t)n_blk * 32 * R;
  const PT* po_blk = part_o + ((int64_t)b * max_splits * n_blk + blk) * (32 * R);
  float mx = -INFINITY, z = 0.0f;
  float acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = 0.0f;
  for (int k0 = kb; k0 < ke; k0 += U) {
    float lk[U];
    raw ok[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int k = k0 + j;
      const uint32_t off = (uint32_t)((k * split_stride + 32 * CW * cg + NV * lane) * sizeof(PT));
      if constexpr (COH) {
        lk[j] = k < ke ? __hip_atomic_load(pl + (int64_t)k * M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                       : -INFINITY;
        if (k < ke) ok[j] = load16_coherent<raw>(po_blk, off);
      } else {
        lk[j] = k < ke ? pl[(int64_t)k * M] : -INFINITY;
        if (k < ke && (!GATE || lk[j] != -INFINITY))
          ok[j] = *reinterpret_cast<const raw*>(reinterpret_cast<const char*>(po_blk) + off);
      }
    }
    float cm = lk[0];
#pragma unroll
    for (int j = 1; j < U; ++j) cm = fmaxf(cm, lk[j]);
    if (cm > mx) {
      const float sc = __expf(mx - cm);   // 0 while mx is still -inf
      z *= sc;
#pragma unroll
      for (int i = 0; i < NV; ++i) acc[i] *= sc;
      mx = cm;
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const bool live = lk[j] != -INFINITY;
      const float w = live ? __expf(lk[j] - mx) : 0.0f;
      z += w;
#pragma unroll
      for (int i = 0; i < NV; ++i) acc[i] = live ? acc[i] + w * PartLoad<PT>::get(ok[j], i) : acc[i];
    }
  }
  bool writer = row_ok;
  if constexpr (WIDE) {
    float* st = s_st + wave * (NV + 2) * 64 + lane;
    st[0] = mx;
    st[64] = z;
#pragma unroll
    for (int i = 0; i < NV; ++i) st[64 * (2 + i)] = acc[i];
    __syncthreads();
    writer = row_ok && wave == 0;
    if (writer) {
      // combine the four states against their common max (a wave without a
      // finite split has max -inf and no weight)
      float mw[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) mw[w] = s_st[w * (NV + 2) * 64 + lane];
      const float mt = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
      mx = mt;
      z = 0.0f;
#pragma unroll
      for (int i = 0; i < NV; ++i) acc[i] = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float* sw = s_st + w * (NV + 2) * 64 + lane;
        const float f = mw[w] == -INFINITY ? 0.0f : __expf(mw[w] - mt);
        z += f * sw[64];
#pragma unroll
        for (int i = 0; i < NV; ++i) acc[i] += f * sw[64 * (2 + i)];
      }
    }
    __syncthreads();                            // s_st is free for the next item
  }
  if (writer) {
    const float inv = z > 0.0f ? 1.0f / z : 0.0f;
    const int t = m / H, h = m - t * H;
    T* o = out + b * out_sb + t * out_st + h * out_sh + CW * cg + 4 * hh;
#pragma unroll
    for (int q4 = 0; q4 < NV / 4; ++q4) {     // value i of the lane is column CW*cg + 8*(i/4) + 4*hh + i%4
      const float v4[4] = {acc[4 * q4] * inv, acc[4 * q4 + 1] * inv, acc[4 * q4 + 2] * inv, acc[4 * q4 + 3] * inv};
      store4<T>(o + 8 * q4, v4);
    }
    if (cg == 0 && hh == 0) lse[(int64_t)b * M + m] = z > 0.0f ? mx + logf(z) : -INFINITY;
  }
}

// The splits of a sequence of n_keys = L + q keys (1 <= n_keys < 2^31):
//  * fixed (tiles_max == 0): splits of split_keys keys; split s covers keys
//    [s split_keys, min(n_keys, (s + 1) split_keys)), ns = ceil(n_keys / split_keys);
//  * adaptive (tiles_max > 0, the key tiles of the longest sequence the launch
//    allows, whose max_splits splits have split_keys keys or fewer): a
//    sequence of T = ceil(n_keys / 32) tiles gets ceil(T max_splits / tiles_max)
//    splits' worth of tiles, tps = ceil(T / that) per split, so every split of
//    every sequence holds about as many tiles as one of the longest sequence;
//    split s covers tiles [s tps, min(T, (s + 1) tps)), ns = ceil(T / tps).
// Splits at or past ns are empty (k_begin >= n_keys).
struct SplitRange {
  int k_begin, k_end, ns;
};
__device__ __forceinline__ SplitRange split_range(int n_keys, int split, int split_keys, int max_splits,
                                                  int tiles_max) {
  SplitRange r;
  if (tiles_max <= 0) {
    r.ns = (int)min((uint32_t)max_splits, (uint32_t)(n_keys - 1) / (uint32_t)split_keys + 1u);
    r.k_begin = split * split_keys;
    r.k_end = min(n_keys, r.k_begin + split_keys);
  } else {
    const uint32_t T = (uint32_t)(n_keys - 1) / kBN + 1u;
    // (32-bit whenever T * max_splits + tiles_max fits: the 64-bit quotient is
    // about 150 scalar instructions)
    const uint32_t ms = (uint32_t)max_splits, tm = (uint32_t)tiles_max;
    const uint32_t want = T <= (0xFFFFFFFFu - tm) / ms
                              ? (T * ms + tm - 1u) / tm
                              : (uint32_t)(((uint64_t)T * (uint64_t)ms + tm - 1) / (uint64_t)tm);
    const uint32_t tps = (T - 1) / max(want, 1u) + 1u;
    r.ns = (int)((T - 1) / tps + 1u);
    r.k_begin = (int)min((uint32_t)split * tps, T) * kBN;
    r.k_end = min(n_keys, (int)(min((uint32_t)(split + 1) * tps, T) * kBN));
  }
  return r;
}

template <typename T, typename PT, int R>
__device__ __forceinline__ void merge_share(const VerifyArgs& a, int b, int rt, int ns, int BM, int unit,
                                            int n_units, float* s_st, int wave, int lane) {
  constexpr int NV = PartLoad<PT>::NV;
  constexpr int n_cg = R / (2 * NV);
  const int blk0 = rt * (BM / 32);
  const int nb = min(BM / 32, a.n_blk - blk0);    // blocks of this row tile holding real rows
  const int n_items = nb * n_cg;
  const PT* po = static_cast<const PT*>(a.part_o);
  T* out = static_cast<T*>(a.out);
  if (a.max_splits > 16) {
    // a workgroup per item: unit = workgroup
    for (int i = unit; i < n_items; i += n_units)
      merge_item<T, PT, true, true>(po, a.part_lse, a.max_splits, ns, a.M, a.H, R, a.n_blk, b, blk0 + i / n_cg,
                                    i % n_cg, out, a.out_sb, a.out_st, a.out_sh, a.lse, s_st, wave, lane);
  } else {
    // a wave per item: unit = workgroup, its waves taking consecutive items
    for (int i = 4 * unit + wave; i < n_items; i += 4 * n_units)
      merge_item<T, PT, false, true>(po, a.part_lse, a.max_splits, ns, a.M, a.H, R, a.n_blk, b, blk0 + i / n_cg,
                                     i % n_cg, out, a.out_sb, a.out_st, a.out_sh, a.lse, s_st, wave, lane);
  }
}

// Work compaction (adaptive splits over several sequences): the (sequence,
// split, row tile) pieces with work are numbered in that order, and
// workgroup i < W (W pieces in all) takes piece xcd_remap(i, W): the working
// workgroups are spread evenly over the XCDs, and the row tiles of one split
// stay together on one XCD (they read the same keys); workgroups i >= W have
// none.  A sequence with an invalid prefix length counts one split (its
// workgroups flag it and write the empty result).  Each wave works it out
// from the prefix lengths itself, 64 sequences per pass.
struct Piece {
  int b, split, rt, L;
  bool work;
};
__device__ __forceinline__ int pieces_of(const VerifyArgs& a, int L) {
  const bool bad = L < 0 || L > a.max_prefix_len || (int64_t)L + a.q > a.capacity;
  return a.n_rt * (bad ? 1 : split_range(L + a.q, 0, a.split_keys, a.max_splits, a.tiles_max).ns);
}
__device__ __forceinline__ Piece compact_piece(const VerifyArgs& a, int lane) {
  Piece pc{0, 0, 0, 0, false};
  int total = 0;
  for (int j0 = 0; j0 < a.B; j0 += 64) {
    const int j = j0 + lane;
    int c = j < a.B ? pieces_of(a, a.prefix_lens[j]) : 0;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d);
    total += __builtin_amdgcn_readfirstlane(c);     // (uniform: the exit below is a uniform branch)
  }
  const int i = blockIdx.x;
  if (i >= total) return pc;
  const int p = xcd_remap(i, total);
  int base = 0;
  for (int j0 = 0; j0 < a.B; j0 += 64) {
    const int j = j0 + lane;
    const int L = j < a.B ? a.prefix_lens[j] : 0;
    const int c = j < a.B ? pieces_of(a, L) : 0;
    int incl = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    const uint64_t past = __ballot(base + incl > p);
    if (past) {
      const int k = __builtin_ctzll(past);
      const int rem = p - (base + __shfl(incl, k) - __shfl(c, k));
      pc.b = j0 + k;
      pc.L = __shfl(L, k);
      pc.split = rem / a.n_rt;
      pc.rt = rem - pc.split * a.n_rt;
      pc.work = true;
      return pc;
    }
    base += __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
  }
  return pc;
}

// One piece of work of a workgroup: row tile rt of sequence b over one key
// range, written as partial `split`.  known: the prefix length L is known
// (else the body loads it).  The key range [k_begin, k_end) and the stream's
// piece count ns are given by the balanced schedule; the other schedules
// take them from split_range.
struct PieceDesc {
  int b, rt, split, L, k_begin, k_end, ns;
  bool known;
};

__device__ __forceinline__ bool len_bad(const VerifyArgs& a, int L) {
  return L < 0 || L > a.max_prefix_len || (int64_t)L + a.q > a.capacity;
}
// key tiles of a sequence of prefix length L (one for an invalid length,
// whose workgroups flag it and write the empty result)
__device__ __forceinline__ int tiles_of(const VerifyArgs& a, int L) {
  return len_bad(a, L) ? 1 : (L + a.q - 1) / kBN + 1;
}
// units of one stream of sequence b: its start-up (piece_units) and its key
// tiles; a sequence with an invalid length is one unit
__device__ __forceinline__ int units_of(const VerifyArgs& a, int L) {
  return len_bad(a, L) ? 1 : a.piece_units + (L + a.q - 1) / kBN + 1;
}

// Work-balanced schedule (stream-K style).  The row tiles of a sequence are
// cut into n_grp groups of `gang` (the last may be short), and each
// (sequence, group) pair is a stream of units: piece_units for the start-up
// its first piece costs, then one per key tile of the sequence.  The
// streams are laid end to end, sequence-major, U units in all, and gang j of
// the launch's G gangs takes units [j A, min(U, (j + 1) A)) with A =
// ceil(U / G), raised so that no stream's key tiles meet more than
// max_splits gangs (A >= ceil(T_max / (max_splits - 1)), T_max the most key
// tiles of a sequence) and capped at span_keys / 32 (then gang j also takes
// the ranges of gangs j + G, j + 2 G, ... after its own).  A range that ends
// inside a stream's start-up units holds no piece of it.  A gang is `gang` workgroups that are consecutive after xcd_remap,
// so they share an XCD and its L2: member m does row tile grp * gang + m of
// every stream the gang's range meets, so the members read the same keys at
// about the same time.  Where a range crosses from one stream into the
// next, its workgroups finish one piece (one partial) and start the next.
// The piece of a stream that gang j does is the stream's partial
// j - floor(r / A), r the stream's first key-tile unit, and a stream has
// floor(last unit / A) - floor(r / A) + 1 of them.  Every wave walks the ranges itself
// from the prefix lengths (64 sequences per pass); all values are uniform.
struct BalWalk {
  int A, U;        // units per gang, units in all (the host keeps U below 2^31)
  int s, e;        // next unit, end of the current range
  int st;          // first unit of the current stream
  int j;           // current gang
  int b, grp, L, T;  // current stream: sequence, row-tile group, prefix length, units
  int member;
};

__device__ __forceinline__ int udiv(int x, int y) { return (int)((uint32_t)x / (uint32_t)y); }

// the stream holding unit w.s
__device__ __forceinline__ void bal_locate(const VerifyArgs& a, BalWalk& w, int lane) {
  int base = 0;     // units of the sequences before this pass's
  for (int j0 = 0; j0 < a.B; j0 += 64) {
    const int j = j0 + lane;
    const int L = j < a.B ? a.prefix_lens[j] : 0;
    const int c = j < a.B ? a.n_grp * units_of(a, L) : 0;
    int incl = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    const uint64_t past = __ballot(base + incl > w.s);
    if (past) {
      const int k = __builtin_ctzll(past);
      w.b = j0 + k;
      w.L = __builtin_amdgcn_readfirstlane(__shfl(L, k));
      w.T = units_of(a, w.L);
      const int sb = __builtin_amdgcn_readfirstlane(base + __shfl(incl, k) - __shfl(c, k));
      w.grp = udiv(w.s - sb, w.T);
      w.st = sb + w.grp * w.T;
      return;
    }
    base += __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
  }
}

// Sets up workgroup blockIdx.x's walk; false if it has no work.
__device__ __forceinline__ bool bal_init(const VerifyArgs& a, BalWalk& w, int lane) {
  int useq = 0;
  int tmax = 1;
  for (int j0 = 0; j0 < a.B; j0 += 64) {
    const int j = j0 + lane;
    const int L = j < a.B ? a.prefix_lens[j] : 0;
    int c = j < a.B ? units_of(a, L) : 0;
    int tm = j < a.B ? tiles_of(a, L) : 1;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      c += __shfl_xor(c, d);
      tm = max(tm, __shfl_xor(tm, d));
    }
    useq += __builtin_amdgcn_readfirstlane(c);
    tmax = max(tmax, __builtin_amdgcn_readfirstlane(tm));
  }
  w.U = a.n_grp * useq;
  const int G = a.gangs;
  int A = udiv(w.U + G - 1, G);
  A = max(A, udiv(tmax + a.max_splits - 2, a.max_splits - 1));
  A = min(A, a.span_keys / kBN);
  w.A = max(A, 1);
  const int u = xcd_remap(blockIdx.x, gridDim.x);
  w.j = udiv(u, a.gang);
  w.member = u - w.j * a.gang;
  if ((int64_t)w.j * w.A >= w.U) return false;
  w.s = w.j * w.A;
  w.e = min(w.U - w.s, w.A) + w.s;
  bal_locate(a, w, lane);
  return true;
}

// The next piece of the walk (pieces of row tiles past the last are
// skipped); false when the workgroup's ranges are done.
__device__ __forceinline__ bool bal_next(const VerifyArgs& a, BalWalk& w, int lane, PieceDesc& pc) {
  while (true) {
    if (w.s >= w.e) {
      w.j += a.gangs;
      if ((int64_t)w.j * w.A >= w.U) return false;
      w.s = w.j * w.A;
      w.e = min(w.U - w.s, w.A) + w.s;
      bal_locate(a, w, lane);
    } else if (w.s >= w.st + w.T) {
      w.st += w.T;
      if (++w.grp == a.n_grp) {
        w.grp = 0;
        ++w.b;
        w.L = ((const __attribute__((address_space(4))) int32_t*)a.prefix_lens)[w.b];
        w.T = units_of(a, w.L);
      }
    }
    const int s0 = w.s;
    const int pe = min(w.e, w.st + w.T);
    w.s = pe;
    const int rt = w.grp * a.gang + w.member;
    const bool bad = len_bad(a, w.L);
    const int rs = w.st + (bad ? 0 : a.piece_units);    // the stream's first key-tile unit
    if (rt >= a.n_rt || pe <= rs) continue;
    const int k0 = max(s0, rs);
    pc.b = w.b;
    pc.rt = rt;
    pc.L = w.L;
    pc.known = true;
    pc.split = udiv(k0, w.A) - udiv(rs, w.A);
    pc.ns = udiv(w.st + w.T - 1, w.A) - udiv(rs, w.A) + 1;
    pc.k_begin = (k0 - rs) * kBN;
    pc.k_end = bad ? 1 : min(w.L + a.q, (pe - rs) * kBN);
    return true;
  }
}

// The merge of one row tile's partials inside the split kernel.  The split
// workgroups of (sequence b, row tile rt) share one 32-bit state word: bits
// 0-15 count arrivals, bits 16-30 count workgroups that gave up waiting, and
// bit 31 is a generation bit.  Partials and their log-sum-exps are stored
// device-coherent (sc1); a workgroup whose waves have all seen their stores
// complete adds one arrival:
//  * the last to arrive (it reads ns - 1 arrivals back) knows every partial
//    is in place; it writes the word back with zero counts and the generation
//    flipped, which both releases the others and leaves the word ready for
//    the next call, then merges its share of the row tile's items, or every
//    item if some workgroup gave up before it arrived;
//  * the others wait, for at most spin_ticks of the 100 MHz clock, for the
//    generation to flip, then merge their share.  A workgroup that runs out
//    of time adds one to the give-up count with a compare-and-swap that only
//    succeeds while the generation has not flipped, and leaves: the last
//    arriver then sees the count and merges everything.  If the swap finds
//    the generation flipped, the workgroup merges its share after all.
// The merge reads the partials with device-coherent loads.  Every workgroup
// leaves after a bounded wait whatever the others do, so the grid always
// drains.  An item is merged by the same code in the same order whoever
// merges it (twice, identically, when the last arriver takes over), so the
// output does not depend on who did.  The wait is short when all split
// workgroups of a row tile are resident at once, which the host ensures by
// fusing only when the grid fits the compute units.  Items: with more than
// sixteen splits in the launch a workgroup per item (its waves sharing the
// splits, as in merge_kernel), otherwise a wave per item.
template <typename T, int R>
__device__ __forceinline__ void fused_merge(const VerifyArgs& a, int b, int rt, int split, int ns, int BM,
                                            float* s_st, int tid) {
  __shared__ int s_mode;
  const int wave = tid >> 6, lane = tid & 63;
  uint32_t* word = reinterpret_cast<uint32_t*>(a.counters) + ((int64_t)b * a.n_rt + rt);
  wait_vmem_lds<0>();                                   // this wave's partial stores are complete
  asm volatile("" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    // mode: 0 = leave, 1 = merge this workgroup's share, 2 = merge every item
    int mode = 1;
    const uint32_t old = __hip_atomic_fetch_add(word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t gen = old & 0x80000000u;
    if ((int)(old & 0xFFFFu) == ns - 1) {
      __hip_atomic_store(word, gen ^ 0x80000000u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old & 0x7FFF0000u) mode = 2;
    } else {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (true) {
        uint32_t v = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((v & 0x80000000u) != gen) break;
        if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) >= a.spin_ticks) {
          // give up, unless the generation flips first
          while ((v & 0x80000000u) == gen &&
                 !__hip_atomic_compare_exchange_strong(word, &v, v + 0x10000u, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT)) {
          }
          if ((v & 0x80000000u) == gen) mode = 0;   // the swap succeeded: registered, leave
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    s_mode = mode;
  }
  __syncthreads();
  asm volatile("" ::: "memory");
  const int mode = s_mode;
  if (mode == 0) return;
  if (a.part_bf16) {
    if (mode == 1) merge_share<T, __bf16, R>(a, b, rt, ns, BM, split, ns, s_st, wave, lane);
    else merge_share<T, __bf16, R>(a, b, rt, ns, BM, 0, 1, s_st, wave, lane);
  } else {
    if (mode == 1) merge_share<T, float, R>(a, b, rt, ns, BM, split, ns, s_st, wave, lane);
    else merge_share<T, float, R>(a, b, rt, ns, BM, 0, 1, s_st, wave, lane);
  }
}

// CS (column split) = 1: the four waves own 32 rows each, all R output
// columns.  CS = 2, for sequences of at most 64 rows (AR decoding and small
// trees): two row blocks of 32, each owned by a pair of waves that compute the
// same scores and softmax and split the R output columns between them.  Each
// wave then holds half the accumulators and does half the value
// MFMAs; the duplicated score MFMAs are spare capacity when the memory stream
// is the bound.
// The kernel's arguments, read again from the kernel argument segment
// through an opaque pointer (the one argument, a VerifyArgs, sits at its
// start): values derived from them are then computed where they are used,
// once per piece, rather than hoisted out of the piece loop and held in
// registers across every piece.
__device__ __forceinline__ VerifyArgs reread_args() {
  typedef const __attribute__((address_space(4))) uint32_t cu32;
  cu32* src = (cu32*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(src));
  static_assert(sizeof(VerifyArgs) % 4 == 0, "argument words");
  uint32_t w[sizeof(VerifyArgs) / 4];
#pragma unroll
  for (int i = 0; i < (int)(sizeof(VerifyArgs) / 4); ++i) w[i] = src[i];
  VerifyArgs a;
  __builtin_memcpy(&a, w, sizeof(VerifyArgs));
  return a;
}

// BAL: the balanced schedule (a workgroup walks several pieces; a separate
// instantiation, so that the one-piece kernels keep their registers).
template <typename T, int R, int P, bool DIRECT, int CS, bool BAL = false>
__global__ __launch_bounds__(kThreads, 1) void verify_split_kernel(VerifyArgs a_in) {
  typedef Mfma<T> MM;
  typedef typename MM::frag frag;
  constexpr int D = R + P;
  constexpr int KW = MM::KW, KMF = MM::KMF;
  constexpr int NCHUNK = D / KMF;             // MFMA steps of the score contraction
  constexpr int NB = R / 32;                  // 32-wide output column blocks
  static_assert(CS >= 1 && CS <= 4, "layout");
  // CS = 3: the 64-row layout with the score contraction split by depth: the
  // two waves of a pair each contract half of the R + P columns, exchange
  // their partial scores through LDS and add them, so no score MFMA is done
  // twice; the softmax is duplicated as in CS = 2 and the values split by
  // columns.
  constexpr bool DS = (CS == 3);
  // CS = 4: 64 rows, two key streams.  Wave w owns row block w / 2 and all R
  // output columns, and takes every other key tile (stream w % 2), so no
  // contraction step is done twice and each tile is read by two waves; the
  // two streams' softmax states and accumulators are combined once, after
  // the last tile.  As in layout 1, the query's rope part is read from LDS
  // every tile.
  constexpr bool KS = (CS == 4);
  constexpr int CSC = DS ? 2 : (KS ? 1 : CS); // column split of the output
  static_assert(!DS || (NCHUNK % 2 == 0 && KW == 8), "depth split: bf16, even contraction steps");
  static_assert(!KS || (KW == 8 && R % KMF == 0), "key streams: bf16");
  constexpr int NQR = NCHUNK - R / KMF;       // rope steps of the score contraction
  // Layouts 1 (at rank 512) and 4 read the query's rope fragments from LDS
  // every tile instead of holding them, which frees the registers the score
  // tile needs while all 256 accumulation registers are taken.
  constexpr bool QPE = KS || (CS == 1 && KW == 8 && NB == 16);
  // query fragments held in registers by one wave (score steps)
  constexpr int NQF = DS ? NCHUNK / 2 : (QPE ? R / KMF : NCHUNK);
  constexpr int NSTEP = QPE ? NCHUNK : NQF;   // score steps of one wave
  constexpr int NBL = NB / CSC;               // output column blocks of one wave
  constexpr int BM = KS ? kBM / 2 : kBM / CSC;    // query rows per workgroup
  constexpr int PV_STEPS = kBN / KMF;         // MFMA steps of the value contraction per tile
  constexpr int RC = R * (int)sizeof(T) / 16; // 16-byte chunks of c_kv per key
  constexpr int PC = P * (int)sizeof(T) / 16; // 16-byte chunks of k_pe per key
  constexpr int LAT_BYTES = kBN * RC * 16;
  constexpr int BUF_BYTES = LAT_BYTES + kBN * PC * 16;
  static_assert(R % 32 == 0 && D % KMF == 0 && (P * sizeof(T)) % 16 == 0, "shape");

  // Ring of NBUF key-tile buffers, NBUF - 1 copies in flight: three where
  // the query's rope fragments (layout 1) or the partial scores (layout 3)
  // also need LDS, four otherwise.  The copies are inline asm the compiler
  // does not track, so one array indexed with constants serves.
  static_assert(NBL < 16 || QPE, "a wave owning all 512 columns reads its rope fragments from LDS");
  constexpr int NBUF = (CS == 1 || DS) ? 3 : 4;
  __shared__ __attribute__((aligned(1024))) char s_tiles[NBUF][BUF_BYTES];
  // vmcnt per tile copy on every wave (a wave that issued more waits a
  // little longer, which is safe).
  constexpr int STAGE_LOADS = min_wave_loads(kBN * RC) + min_wave_loads(kBN * PC);
  static_assert(STAGE_LOADS * (NBUF - 2) < 64, "vmcnt range");
  __shared__ int s_dead;
  // per-wave pointer-doubling area when the masks are derived from parents
  // (one area, run by wave 0, in the key-stream layout, whose LDS is full)
  constexpr int NVA = KS ? 1 : kThreads / kWave;
  __shared__ uint64_t s_vm[NVA][2 * KDT_MAX_Q_LEN];
  __shared__ int s_vj[NVA][KDT_MAX_Q_LEN];
  // the rope part of each row block's query fragments, one 16-byte fragment
  // per (row block, step, lane)
  __shared__ __attribute__((aligned(16))) char s_qpe[QPE ? (BM / 32) * NQR * 64 * 16 : 16];
  // depth split: each wave's partial score tile, 16 floats per lane
  __shared__ __attribute__((aligned(16))) f32x4 s_sx[DS ? 4 * kThreads : 1];

  // Logical work unit u: the row tiles of one (sequence, split) group are
  // consecutive (they read the same keys, and xcd_remap keeps consecutive
  // units on one XCD, sharing its L2); the groups are visited in the order
  // g = g' * group_mul mod (B * max_splits), group_mul coprime to the group
  // count, so that each XCD's block of units mixes sequences and splits
  // (with adaptive splits a short sequence's high splits have no work).
  // Pieces: one per workgroup, except in the balanced schedule, where a
  // workgroup walks its ranges piece by piece (the workgroup meets at a
  // barrier between pieces, so that no wave reuses LDS another still reads).
  // The walk's state lives in LDS between pieces (two slots, by piece
  // parity: every wave reads the current one after the barrier, the first
  // thread writes the next), so no register holds it across a piece.
  static_assert(!BAL || (!DIRECT && (CS == 1 || CS == 2)), "balanced schedule: layouts 1 and 2, partials");
  constexpr bool SCORE_VGPR = KW == 8 && !(BAL && CS == 2);
  __shared__ BalWalk s_walk[BAL ? 2 : 1];
  bool more = true;
  if constexpr (BAL) {
    BalWalk w0;
    more = bal_init(a_in, w0, threadIdx.x & 63);
    if (threadIdx.x == 0) s_walk[0] = w0;
    __syncthreads();
  }
#pragma unroll 1
  for (int iter = 0; BAL ? more : iter < 1; ++iter) {
    // Balanced schedule: the arguments and the thread index are taken afresh
    // for every piece (the index through an opaque zero), so that what the
    // body derives from them is computed inside the loop, not hoisted out of it
    // and held in registers across every piece.
    // (the one-piece kernels read the argument itself, whose loads the
    // compiler may repeat instead of holding their values)
    VerifyArgs a_piece;
    if constexpr (BAL) a_piece = reread_args();
    const VerifyArgs& a = BAL ? a_piece : a_in;
    int opaque0 = 0;
    if constexpr (BAL) asm volatile("s_mov_b32 %0, 0" : "=s"(opaque0));
    const int tid = (int)threadIdx.x + opaque0;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    PieceDesc pc;
    if constexpr (BAL) {
      if (iter > 0) __syncthreads();
      BalWalk walk;
      {
        const BalWalk& sw = s_walk[iter & 1];
        walk.A = __builtin_amdgcn_readfirstlane(sw.A);
        walk.U = __builtin_amdgcn_readfirstlane(sw.U);
        walk.s = __builtin_amdgcn_readfirstlane(sw.s);
        walk.e = __builtin_amdgcn_readfirstlane(sw.e);
        walk.st = __builtin_amdgcn_readfirstlane(sw.st);
        walk.j = __builtin_amdgcn_readfirstlane(sw.j);
        walk.b = __builtin_amdgcn_readfirstlane(sw.b);
        walk.grp = __builtin_amdgcn_readfirstlane(sw.grp);
        walk.L = __builtin_amdgcn_readfirstlane(sw.L);
        walk.T = __builtin_amdgcn_readfirstlane(sw.T);
        walk.member = __builtin_amdgcn_readfirstlane(sw.member);
      }
      if (!bal_next(a, walk, lane, pc)) break;
      if (tid == 0) s_walk[(iter + 1) & 1] = walk;
    } else {
      more = false;
      if (a.compact) {
        const Piece cp = compact_piece(a, lane);
        if (!cp.work) return;
        pc.rt = __builtin_amdgcn_readfirstlane(cp.rt);
        pc.split = __builtin_amdgcn_readfirstlane(cp.split);
        pc.b = __builtin_amdgcn_readfirstlane(cp.b);
        pc.L = __builtin_amdgcn_readfirstlane(cp.L);
        pc.known = true;
      } else {
        const int u = xcd_remap(blockIdx.x, gridDim.x);
        pc.rt = u % a.n_rt;
        // (32-bit arithmetic whenever the product cannot overflow: the 64-bit
        // remainder is about 150 scalar instructions before the first copy)
        const int n_grp = a.B * a.max_splits, gq = u / a.n_rt;
        const int g = n_grp <= 46340 ? (int)((uint32_t)gq * (uint32_t)a.group_mul % (uint32_t)n_grp)
                                     : (int)((int64_t)gq * a.group_mul % n_grp);
        pc.split = g % a.max_splits;
        pc.b = g / a.max_splits;
        pc.L = 0;
        pc.known = false;
      }
      pc.k_begin = pc.k_end = pc.ns = 0;
    }
    const int rt = pc.rt, split = pc.split, b = pc.b;
    const int r = lane & 31, hh = lane >> 5;
    // row block, output column half (and depth half), key stream
    const int rb = KS ? (wave >> 1) : wave / CSC, chalf = KS ? 0 : wave % CSC, kp = KS ? (wave & 1) : 0;
    const int c0 = DS ? chalf * NQF : 0;          // first score step of this wave
    const int m = rt * BM + rb * 32 + r;        // this lane's query row
    const bool row_ok = m < a.M;
    const int t = row_ok ? m / a.H : 0;
    const int h = row_ok ? m - t * a.H : 0;

    // Start-up order: the speculative copies of the first two key tiles, so
    // the key stream starts at once, then the query fragments and visibility
    // words, then the prefix length (a scalar load: the index is uniform, so
    // waiting for it waits for no vector load).  All four latencies overlap.
    // the split's first key as for a sequence of the longest length the
    // launch allows (right for it and for every split of fixed size; the
    // speculative copies below use it)
    const bool L_bad_known = pc.known && len_bad(a, pc.L);
    const int k_spec = !pc.known ? split * a.split_keys
                       : L_bad_known ? 0
                       : BAL ? pc.k_begin
                             : split_range(pc.L + a.q, split, a.split_keys, a.max_splits, a.tiles_max).k_begin;
    int k_begin = k_spec;
    const char* kv_lat = reinterpret_cast<const char*>(a.c_kv) + (b * a.c_kv_sb) * (int64_t)sizeof(T);
    const char* kv_pe = reinterpret_cast<const char*>(a.k_pe) + (b * a.k_pe_sb) * (int64_t)sizeof(T);
    const uint32_t lat_ss = (uint32_t)(a.c_kv_ss * (int64_t)sizeof(T));
    const uint32_t pe_ss = (uint32_t)(a.k_pe_ss * (int64_t)sizeof(T));
    // One buffer descriptor per region for the whole split, so that a tile
    // copy only adds its row offset.  It spans the split's rows below the cache
    // capacity (the host keeps split_keys rows of either region under 2^31
    // bytes); every row a copy reads is one of them.
    auto span_of = [&](int kb) {
      return max((int64_t)0, min((int64_t)a.span_keys, a.capacity - (int64_t)kb));
    };
    i32x4 rs_lat = make_rsrc(kv_lat + (int64_t)k_begin * lat_ss, (uint32_t)(span_of(k_begin) * lat_ss));
    i32x4 rs_pe = make_rsrc(kv_pe + (int64_t)k_begin * pe_ss, (uint32_t)(span_of(k_begin) * pe_ss));
    // Copy of key tile `tile` (first key k_begin + tile * kBN) into the tile
    // buffer at LDS address lds, with its first `nrows` rows real; later rows
    // repeat row nrows - 1.
    auto stage_rows = [&](int tile, uint32_t lds, int nrows) {
      const uint32_t r0 = (uint32_t)(tile * kBN);
      stage_region<kBN, RC>(rs_lat, r0 * lat_ss, lat_ss, nrows, lds, wave, lane);
      stage_region<kBN, PC>(rs_pe, r0 * pe_ss, pe_ss, nrows, lds + LAT_BYTES, wave, lane);
    };
    // Speculative copies of the first two tiles as if the split were full:
    // rows below the cache capacity are always inside the caller's buffer, so
    // this is safe before the prefix length is known; it is right whenever the
    // split really covers both tiles (every split but a sequence's last).
    const bool spec = (int64_t)k_begin + 2 * kBN <= a.capacity;
    // Parents (when the masks are derived here) are loaded first, so that by
    // the time any later copy has been waited for they have landed too.
    int par_v[2] = {-1, -1};
    if (a.parents) {
      const int32_t* pp = a.parents + (int64_t)b * a.q;
      par_v[0] = lane < a.q ? pp[lane] : -1;
      par_v[1] = lane + 64 < a.q ? pp[lane + 64] : -1;
    }
    if (spec) {
      stage_rows(0, lds_addr(s_tiles[0]), kBN);
      stage_rows(1, lds_addr(s_tiles[1]), kBN);
    }

    // The query fragments and visibility words do not depend on the prefix
    // length.  Padding rows (m >= M) load token 0 / head 0: an output column of
    // either contraction depends only on its own query column, and padding rows
    // are never written, so no masking is needed.
    //
    // In the 64-row layout (bf16) the workgroup's query rows are copied like
    // two key tiles, into the two ring buffers the first tiles leave free, and
    // each wave then reads its fragments with the score operand's LDS pattern:
    // 1 KB contiguous per copy instead of 32 scattered rows per load.
    constexpr bool Q_VIA_LDS = (CS == 2 || KS) && (KW == 8) && (NBUF == 4);
    static_assert(!Q_VIA_LDS || BM == 2 * kBN, "query staging: two 32-row blocks per workgroup");
    const bool q_lds = Q_VIA_LDS && a.q_rows_uniform;
    frag qf[NQF];
    if (q_lds) {
      const uint32_t ql_ss = (uint32_t)(a.q_lat_sh * (int64_t)sizeof(T));
      const uint32_t qp_ss = (uint32_t)(a.q_pe_sh * (int64_t)sizeof(T));
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int row0 = rt * BM + blk * kBN;
        const int nr = min(kBN, a.M - row0);    // rows of this block that exist
        const int base_row = nr > 0 ? row0 : rt * BM;
        const int nrows = nr > 0 ? nr : 1;
        const char* ql = reinterpret_cast<const char*>(a.q_lat) +
                         (b * a.q_lat_sb + (int64_t)base_row * a.q_lat_sh) * (int64_t)sizeof(T);
        const char* qp = reinterpret_cast<const char*>(a.q_pe) +
                         (b * a.q_pe_sb + (int64_t)base_row * a.q_pe_sh) * (int64_t)sizeof(T);
        stage_region<kBN, RC>(make_rsrc(ql, (uint32_t)nrows * ql_ss), 0, ql_ss, nrows, lds_addr(s_tiles[2 + blk]),
                              wave, lane);
        stage_region<kBN, PC>(make_rsrc(qp, (uint32_t)nrows * qp_ss), 0, qp_ss, nrows,
                              lds_addr(s_tiles[2 + blk]) + LAT_BYTES, wave, lane);
      }
    } else {
      const T* ql = reinterpret_cast<const T*>(a.q_lat) + b * a.q_lat_sb + t * a.q_lat_st + h * a.q_lat_sh;
      const T* qp = reinterpret_cast<const T*>(a.q_pe) + b * a.q_pe_sb + t * a.q_pe_st + h * a.q_pe_sh;
#pragma unroll
      for (int j = 0; j < NQF; ++j) {
        const int c = c0 + j;
        if (c < R / KMF) qf[j] = *reinterpret_cast<const frag*>(ql + c * KMF + hh * KW);
        else qf[j] = *reinterpret_cast<const frag*>(qp + (c * KMF - R) + hh * KW);
      }
      if constexpr (QPE) {
        // the rope fragments go to LDS (one wave of each row block writes them)
        if (kp == 0) {
#pragma unroll
          for (int i = 0; i < NQR; ++i)
            *reinterpret_cast<frag*>(s_qpe + ((rb * NQR + i) * 64 + lane) * 16) =
                *reinterpret_cast<const frag*>(qp + i * KMF + hh * KW);
        }
      }
    }
    uint64_t vw0 = ~0ull, vw1 = ~0ull;
    if (row_ok && a.vis) {
      const uint64_t* vr = a.vis + ((int64_t)b * a.q + t) * a.W;
      vw0 = vr[0];
      vw1 = a.W > 1 ? vr[1] : 0ull;
    }
    const int L = pc.known ? pc.L : ((const __attribute__((address_space(4))) int32_t*)a.prefix_lens)[b];

    const bool bad = len_bad(a, L);
    const int N = L + a.q;
    SplitRange sr;
    if (BAL) {
      sr.k_begin = pc.k_begin;
      sr.k_end = pc.k_end;
      sr.ns = pc.ns;
    } else {
      sr = split_range(bad ? 1 : N, split, a.split_keys, a.max_splits, a.tiles_max);
    }
    k_begin = sr.k_begin;
    // (compaction and the balanced schedule run no workgroup for the splits a
    // sequence does not use: the workgroups of its first split mark them empty)
    const bool fill_unused = BAL || a.compact;

    if (bad || k_begin >= N) wait_vmem_lds<0>();   // no copy may outlive the workgroup
    if (bad) {
      // skipped sequence: zero output, lse = -inf (direct) or an empty partial
      if (tid == 0 && rt == 0 && split == 0) flag_seq(a.seq_status, b, KDT_SEQ_BAD_LEN);
      if (row_ok && hh == 0 && chalf == 0 && (!a.fuse || split == 0)) {
        if (DIRECT || a.fuse) {
          a.lse[(int64_t)b * a.M + m] = -INFINITY;
          T* o = reinterpret_cast<T*>(a.out) + b * a.out_sb + t * a.out_st + h * a.out_sh;
          for (int d = 0; d < R; ++d) o[d] = (T)0.0f;
        } else {
          // (a skipped sequence has one split there: it writes them all)
          for (int k = split; k < (fill_unused ? a.max_splits : split + 1); ++k)
            a.part_lse[((int64_t)b * a.max_splits + k) * a.M + m] = -INFINITY;
        }
      }
      continue;
    }
    if (!DIRECT && fill_unused && !a.fuse && split == 0 && row_ok && hh == 0 && chalf == 0 && kp == 0) {
      for (int k = sr.ns; k < a.max_splits; ++k) a.part_lse[((int64_t)b * a.max_splits + k) * a.M + m] = -INFINITY;
    }
    if (k_begin >= N) {
      // this split does not exist for sequence b: an empty partial, so that a
      // merge over all max_splits splits is always right
      if (!DIRECT && !a.fuse && row_ok && hh == 0 && chalf == 0 && kp == 0)
        a.part_lse[((int64_t)b * a.max_splits + split) * a.M + m] = -INFINITY;
      continue;
    }
    const int k_end = sr.k_end;
    const int n_tiles = (k_end - k_begin + kBN - 1) / kBN;
    const bool spec_ok = spec && k_begin == k_spec && k_begin + 2 * kBN <= k_end;
    if (k_begin != k_spec) {
      // (adaptive splits of a shorter sequence: the speculative copies read
      // other rows, and are waited for and replaced below)
      rs_lat = make_rsrc(kv_lat + (int64_t)k_begin * lat_ss, (uint32_t)(span_of(k_begin) * lat_ss));
      rs_pe = make_rsrc(kv_pe + (int64_t)k_begin * pe_ss, (uint32_t)(span_of(k_begin) * pe_ss));
    }

    auto stage = [&](int tile, uint32_t lds) { stage_rows(tile, lds, min(kBN, k_end - (k_begin + tile * kBN))); };
    // The same copy, one wave-load at a time (pieces 0 .. NPIECE - 1), so that
    // the copies can be issued between value MFMAs: a wave waiting for the
    // texture unit to accept a copy then still has MFMAs in flight.
    constexpr int LAT_PIECES = region_wave_loads<kBN, RC>();
    constexpr int NPIECE = LAT_PIECES + region_wave_loads<kBN, PC>();
    auto stage_piece = [&](int tile, int nrows, uint32_t lds, int piece) __attribute__((always_inline)) {
      const uint32_t r0 = (uint32_t)(tile * kBN);
      if (piece < LAT_PIECES)
        stage_one<kBN, RC, KS>(rs_lat, r0 * lat_ss, lat_ss, nrows, lds, wave, lane, piece);
      else
        stage_one<kBN, PC>(rs_pe, r0 * pe_ss, pe_ss, nrows, lds + LAT_BYTES, wave, lane, piece - LAT_PIECES);
    };



    // Per-lane LDS byte offsets inside a tile buffer (bf16 only; the fp32 path
    // computes its addresses inline).
    //  * score operand, step c: chunk 2c + hh of key r.  With a swizzle over LSW
    //    chunks, 2c + hh = LSW * (c / QB) + (2 * (c % QB) + hh) for QB = LSW / 2
    //    and the swizzle only touches the second part, so the address is
    //    qk_lat[c % QB] + 16 * LSW * (c / QB).
    //  * value operand, transposing read: in each 16-lane group, lane 4e + q
    //    loads columns d0 + 4q .. d0 + 4q + 3 of key k_e and lane j then holds
    //    column d0 + j of keys k_0..k_3.  Operand row d = 32 * db + r; slots 0-3
    //    are keys c_row(8c + 0..3, hh), slots 4-7 keys c_row(8c + 4..7, hh).
    //    The 16-byte chunk is 4 * db + x with x < 4, and (4 db + x) ^ s =
    //    4 (db ^ s2) + (x ^ s01) for s2 = s >> 2, s01 = s & 3; db ^ s2 only
    //    changes the low two bits of db.  The keys are 16c + (8 half + 4 hh +
    //    e) and the swizzle depends on the key modulo 16 only, so c moves the
    //    address by whole 16-key blocks: pv_base[half][db % 4] + 64 * db +
    //    c * (16 rows of the region).
    constexpr int LSW = (RC % 16 == 0) ? 16 : 8;
    constexpr int QB = LSW / 2;
    int qk_lat[QB], qk_pe[4];
    int pv_base[2][4];
    if constexpr (KW == 8) {
      static_assert(P / KMF <= 4 && RC % 8 == 0, "bf16 score addressing");
      const int sr = swz_of<RC>(r);
#pragma unroll
      for (int j = 0; j < QB; ++j) qk_lat[j] = r * RC * 16 + (((2 * j + hh) ^ sr) << 4);
#pragma unroll
      for (int j = 0; j < 4; ++j)   // rope region: chunk 2j + hh exists only while it is < PC
        qk_pe[j] = LAT_BYTES + region_off<PC>(r, (2 * j + hh) < PC ? (2 * j + hh) : 0);
      const int g = lane >> 4, sl = lane & 15;
      const int e = sl >> 2, qd = sl & 3;
      const int x = 2 * (g & 1) + (qd >> 1);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int k = c_row(4 * half + e, hh);
        const int sk = swz_of<RC>(k), s2 = sk >> 2, s01 = sk & 3;
        const int base = k * RC * 16 + ((x ^ s01) << 4) + 8 * (qd & 1);
#pragma unroll
        for (int d4 = 0; d4 < 4; ++d4) pv_base[half][d4] = base + 64 * ((d4 ^ s2) - d4);
      }
    }

    // Visibility words from parent pointers, only where this split reaches the
    // tree (keys L .. N - 1): every wave runs the pointer doubling for the
    // sequence in its own LDS area and reads its tokens' rows.
    auto derive_vis = [&]() {
      if (!a.parents || k_end <= L) return;
      uint64_t m0[2], m1[2];
      const int va = KS ? 0 : wave;
      if (!KS || wave == 0) {
        const bool bad_tree = wave_ancestor_masks(par_v, a.q, s_vm[va], s_vj[va], lane, m0, m1);
        if (__any(bad_tree) && lane == 0 && wave == 0) flag_seq(a.seq_status, b, KDT_SEQ_BAD_TREE);
      }
      if constexpr (KS) {
        wait_lds();
        tile_barrier();
      }
      if (row_ok) {
        vw0 = s_vm[va][2 * t];
        vw1 = s_vm[va][2 * t + 1];
      }
    };

    if constexpr (Q_VIA_LDS) {
      if (q_lds) {
        // the query copies (and the first tiles, issued before them) have landed
        wait_vmem_lds<0>();
        tile_barrier();
        derive_vis();
        const char* qbuf = s_tiles[2 + rb];
#pragma unroll
        for (int c = 0; c < NCHUNK; ++c) {
          const char* src = (c < R / KMF) ? qbuf + qk_lat[c % QB] + 16 * LSW * (c / QB) : qbuf + qk_pe[c - R / KMF];
          if constexpr (KS) {
            if (c < NQF) qf[c] = *reinterpret_cast<const frag*>(src);
            else if (kp == 0)
              *reinterpret_cast<frag*>(s_qpe + ((rb * NQR + (c - NQF)) * 64 + lane) * 16) =
                  *reinterpret_cast<const frag*>(src);
          } else {
            qf[c] = *reinterpret_cast<const frag*>(src);
          }
        }
        // every wave has its fragments before the buffers take key tiles again
        wait_vmem_lds<0>();
        tile_barrier();
      }
    }
    if (!q_lds) derive_vis();

    f32x16 acc[NBL];
#pragma unroll
    for (int i = 0; i < NBL; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;
    // Softmax state of this lane's row (log2 domain).  m_ref is the reference
    // the weights are taken against: fixed at the first tile with a visible key,
    // it never moves while weights stay below 2^kRefSlack, so the accumulators
    // are never rescaled.  m_max is the true running max.  If some row's max
    // outgrows its reference by more than that, the wave's accumulation is void
    // ("dead"): it keeps running its tiles (the copy schedule is shared by all
    // waves) and tracking m_max, then redoes the split once with m_ref = m_max
    // (the exact max), which cannot trigger again, discarding what it summed.
    float m_ref = -INFINITY, m_max = -INFINITY;
    float l_run = 0.0f;           // this lane's share of sum_j exp2(s_j - m_ref)
    bool dead = false;            // wave-uniform

    // One key tile: scores, softmax, value contraction.  `buf` is the tile's
    // ring buffer; the tile's first key is kt.  The copy of the first st_rows
    // rows of tile st_tile into st_buf is issued piece by piece between the
    // value MFMAs.
    // Key streams: the next pair of tiles (copied between this step's score
    // MFMAs; rows 0 = no such tile).
    int ks_t0 = 0, ks_t1 = 0, ks_r0 = 0, ks_r1 = 0;
    // Key streams: accumulator block db of stream kp holds output column block
    // col_block(db) = (db + 8 kp) mod 16, so that every wave keeps blocks 0-7
    // and hands blocks 8-15 to its partner at the end (register indices fixed
    // at compile time on both streams); the value operand of block db is read
    // at LDS offset 64 db + rot_off[db >= 8] instead of 64 col_block(db).
    const int rot_off[2] = {512 * kp, -512 * kp};
    auto col_block = [&](int db) { return KS ? ((db + 8 * kp) & 15) : chalf * NBL + db; };
    uint32_t ks_b0 = 0, ks_b1 = 0;          // (LDS addresses)
    auto tile_body = [&](const int tile, const char* buf, const int st_tile, const int st_rows, uint32_t st_buf)
                         __attribute__((always_inline)) {
      const int kt = k_begin + tile * kBN;
      // ---- scores S^T[key][row]: A = K tile (the lane's key is r), B = Q^T.
      // The K fragments are read QPF steps ahead of the MFMA chain.
      auto score_src = [&](int c) __attribute__((always_inline)) -> const char* {
        if constexpr (KW == 8) {
          // bf16: step c reads 16-byte chunk 2c + hh of the row
          if (c < R / KMF) return buf + qk_lat[c % QB] + 16 * LSW * (c / QB);
          return buf + qk_pe[c - R / KMF];
        } else {
          const int byte = (c * KMF + hh * KW) * (int)sizeof(T);   // byte offset inside the row
          if (c < R / KMF) return buf + region_off<RC>(r, byte >> 4) + (byte & 15);
          return buf + LAT_BYTES + region_off<PC>(r, (byte >> 4) - RC) + (byte & 15);
        }
      };
      // (key streams hold no accumulator block in LDS, so their scores take
      // registers and the operand queues are shorter)
      constexpr int QPF0 = QPE ? 2 : KDT_SCORE_PREFETCH;
      constexpr int QPF = NSTEP < QPF0 ? NSTEP : QPF0;
      frag kf[QPF];
#pragma unroll
      for (int j = 0; j < QPF; ++j) kf[j] = *reinterpret_cast<const frag*>(score_src(c0 + j));
      // this row block's rope fragments of the query, read from LDS QPF steps
      // before their MFMA
      auto qpe_src = [&](int i) { return reinterpret_cast<const frag*>(s_qpe + ((rb * NQR + i) * 64 + lane) * 16); };
      frag qq[QPE ? QPF : 1];
      f32x16 s;
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = 0.0f;
      // (bf16: the tile stays in VGPRs; see Mfma<__bf16>::mma_acc_v.  Not in
      // the balanced 64-row kernel, where the compiler parks query fragments in
      // accumulation registers and copies them back right before their MFMA.)
      auto score_mma = [&](const frag& x, const frag& y, int j) __attribute__((always_inline)) {
        if constexpr (SCORE_VGPR) {
          if (j == 0) s = MM::mma_first_v(x, y);
          else MM::mma_acc_v(x, y, s);
        } else {
          s = MM::mma(x, y, s);
        }
      };
#pragma unroll
      for (int j = 0; j < NSTEP; ++j) {
        const frag cur = kf[j % QPF];
        if (j + QPF < NSTEP) kf[j % QPF] = *reinterpret_cast<const frag*>(score_src(c0 + j + QPF));
        if constexpr (QPE) {
          static_assert(!QPE || NQF >= QPF, "rope fragments are queued behind the register ones");
          // the slot refilled now is the one this step consumes: take it first
          const frag qcur = j < NQF ? qf[j < NQF ? j : 0] : qq[j % QPF];
          if (j + QPF >= NQF && j + QPF < NSTEP) qq[(j + QPF) % QPF] = *qpe_src(j + QPF - NQF);
          score_mma(cur, qcur, j);
        } else {
          score_mma(cur, qf[j], j);
        }
        fence_mem_mfma();
        if constexpr (KS) {
          // the next pair's copies, one wave-load at a time between these MFMAs
          constexpr int NP2 = 2 * NPIECE;
#pragma unroll
          for (int pc = j * NP2 / NSTEP; pc < (j + 1) * NP2 / NSTEP; ++pc) {
            if (pc < NPIECE) stage_piece(ks_t0, ks_r0, ks_b0, pc);
            else stage_piece(ks_t1, ks_r1, ks_b1, pc - NPIECE);
          }
        }
      }
      if constexpr (SCORE_VGPR) MM::score_ready(s);
      if constexpr (DS) {
        // add the partner's half of the contraction (the pair's waves hold the
        // same rows and keys; a + b is the same on both)
#pragma unroll
        for (int g = 0; g < 4; ++g) s_sx[(wave * 4 + g) * 64 + lane] = f32x4{s[4 * g], s[4 * g + 1], s[4 * g + 2], s[4 * g + 3]};
        wait_lds();
        tile_barrier();
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 o = s_sx[((wave ^ 1) * 4 + g) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) s[4 * g + e] += o[e];
        }
      }
      // Value operand of contraction step c (16 keys), output block db.
      auto value_frag = [&](int c, int db) __attribute__((always_inline)) -> frag {
        if constexpr (KW == 1) {
          // fp32: lane (r, hh) needs V[key c_row(c, hh)][32*db + r]
          const int col = ((chalf * NBL + db) * 32 + r) * (int)sizeof(T);
          return *reinterpret_cast<const T*>(buf + region_off<RC>(c_row(c, hh), col >> 4) + (col & 15));
        } else {
          // bf16: two transposing reads (lane bases computed before the loop)
          const int dg = chalf * NBL + db;      // output column block (key streams: rotated, below)
          const int o = (KS ? 64 * db + rot_off[db >= NBL / 2] : 64 * dg) + c * 16 * RC * 16;
          const bf16x4 lo = lds_read_tr16(buf + pv_base[0][dg & 3] + o);
          const bf16x4 hi = lds_read_tr16(buf + pv_base[1][dg & 3] + o);
          return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      };
      constexpr int STEPS = PV_STEPS * NBL;
      constexpr int VPF = STEPS < KDT_VALUE_PREFETCH ? STEPS : KDT_VALUE_PREFETCH;
      // The first value operands are requested now, so their LDS latency
      // passes during the softmax instead of stalling the first value MFMA.
      frag vq[VPF + 1];
#pragma unroll
      for (int i = 0; i < VPF; ++i) vq[i] = value_frag(i / NBL, i % NBL);

      // ---- online softmax for this lane's row (16 of the tile's 32 keys)
      // Raw scores; the scale (positive) is applied to the row max and folded
      // into each weight's exponent, one fused multiply-add per weight.
      float sv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) sv[v] = s[v];
      if (kt + kBN > L || kt + kBN > k_end) {   // only tiles reaching the tree or the split end
        // (an empty volatile asm: without it the compiler turns this branch
        // into selects that every tile then executes, some 200 instructions
        // between the score and the value MFMAs)
        asm volatile("");
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kk = kt + c_row(v, hh);
          const int uu = kk - L;                                  // tree node if >= 0
          const uint64_t w = uu < 64 ? vw0 : vw1;
          const bool tree_ok = uu < 0 || ((w >> (uu & 63)) & 1ull);
          sv[v] = (kk < k_end && tree_ok) ? sv[v] : -INFINITY;
        }
      }
      auto tile_max = [&]() __attribute__((always_inline)) {
        float x = sv[0];
#pragma unroll
        for (int v = 1; v < 16; ++v) x = fmaxf(x, sv[v]);
        return xhalf_max(x) * a.scale_log2;
      };
      // Only tiles where some row of the wave still lacks its reference take
      // this (uniform) branch: the row's running max, this tile included, sets
      // it.  Elsewhere the weights depend on the fixed reference alone.
      if (__any(m_ref == -INFINITY)) {
        const float mx0 = tile_max();
        if (m_ref == -INFINITY) m_ref = fmaxf(m_max, mx0);   // first visible key of this row
      }
      const float m_use = (m_ref == -INFINITY) ? 0.0f : m_ref;
      float p[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[v], a.scale_log2, -m_use));
        l_run += p[v];
      }
      // The running max and the check against the reference feed no weight of
      // this tile, and no branch: they can overlap the value MFMAs.  A wave
      // whose scores outgrow its reference records it in `dead`, which is read
      // after the last tile.
      m_max = fmaxf(m_max, tile_max());
      dead = dead || __any(m_max > m_ref + kRefSlack);

      // ---- O^T[d][row] += V^T[d][key] * P^T[key][row]; the value operand of
      // step i + VPF is read while step i's MFMA is issued (the first VPF were
      // requested before the softmax).
      frag pfr[PV_STEPS];
#pragma unroll
      for (int c = 0; c < PV_STEPS; ++c) pfr[c] = MM::pack(p + c * KW);
#pragma unroll
      for (int i = 0; i < STEPS; ++i) {
        const int c = i / NBL, db = i % NBL;
        if (i + VPF < STEPS) vq[(i + VPF) % (VPF + 1)] = value_frag((i + VPF) / NBL, (i + VPF) % NBL);
        acc[db] = MM::mma(vq[i % (VPF + 1)], pfr[c], acc[db]);
        fence_mem_mfma();
        // copy pieces [i * NPIECE / STEPS, (i + 1) * NPIECE / STEPS) follow this MFMA
        if constexpr (!KS) {
#pragma unroll
          for (int pc = i * NPIECE / STEPS; pc < (i + 1) * NPIECE / STEPS; ++pc)
            stage_piece(st_tile, st_rows, st_buf, pc);
        }
      }
    };

    if (tid == 0) s_dead = 0;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
      if (pass == 1) {
        if (dead) s_dead = 1;
        __syncthreads();
        if (s_dead == 0) break;                 // common case: no redo
        // Depth split: every wave takes part in the score exchange (a
        // workgroup barrier), so all waves redo the split; rows that did not
        // outgrow their reference recompute the same sums.
        if (dead || DS) {
#pragma unroll
          for (int i = 0; i < NBL; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;
          l_run = 0.0f;
          if (dead) m_ref = m_max;
        }
      }
      const bool compute = (pass == 0) || dead || DS;
      dead = false;
      // Tiles rotate through the NBUF buffers: the step for tile t waits for its
      // copy and computes, issuing between its value MFMAs the copy of tile
      // t + NBUF - 1 into the buffer the previous step has finished reading.
      // Every step issues exactly one copy: once no tile is left, a dummy copy
      // (row 0 of tile t, re-read into every row) goes to that buffer, which no
      // later tile uses.  So exactly NBUF - 2 copies are always younger than the
      // one a step waits for, and one wait count serves every step.
      auto wait_tile = [&]() __attribute__((always_inline)) {
        wait_vmem_lds<STAGE_LOADS * (NBUF - 2)>();
        tile_barrier();
      };
      if constexpr (KS) {
        // Key streams: step s computes tiles 2s (waves of stream 0) and 2s + 1
        // (stream 1) from one buffer pair while the next pair's copies go to
        // the other pair of buffers, which the step before has finished
        // reading.  Each step waits for all of its own copies and meets the
        // workgroup at one barrier, after which every copy of the pair has
        // landed and every wave is done with the previous pair.
        if (pass == 0 && spec_ok) {
          wait_vmem_lds<0>();
        } else {
          wait_vmem_lds<0>();
          stage(0, lds_addr(s_tiles[0]));
          if (n_tiles > 1) stage(1, lds_addr(s_tiles[1]));
        }
        const int n_steps = (n_tiles + 1) / 2;
        auto tile_rows = [&](int tt) { return tt < n_tiles ? min(kBN, k_end - (k_begin + tt * kBN)) : 0; };
#pragma unroll 1
        for (int s0 = 0; s0 < n_steps; s0 += 2) {
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) {
            const int st = s0 + hs;
            if (st >= n_steps) break;
            wait_vmem_lds<0>();
            tile_barrier();
            // the next pair; past the last tile a dummy copy (row 0 of tile 0,
            // always inside the split) goes to a buffer no later step reads,
            // so the copies between the score MFMAs need no branch
            const int r0 = tile_rows(2 * st + 2), r1 = tile_rows(2 * st + 3);
            ks_t0 = r0 > 0 ? 2 * st + 2 : 0;
            ks_t1 = r1 > 0 ? 2 * st + 3 : 0;
            ks_r0 = r0 > 0 ? r0 : 1;
            ks_r1 = r1 > 0 ? r1 : 1;
            ks_b0 = lds_addr(s_tiles[2 - 2 * hs]);
            ks_b1 = lds_addr(s_tiles[3 - 2 * hs]);
            const int tt = 2 * st + kp;
            if (compute && tt < n_tiles) {
              tile_body(tt, s_tiles[2 * hs + kp], 0, 0, 0u);
            } else {
              stage_rows(ks_t0, ks_b0, ks_r0);
              stage_rows(ks_t1, ks_b1, ks_r1);
            }
          }
        }
        wait_vmem_lds<0>();
        continue;
      }
      // The first tile, the query fragments and the visibility words are all
      // waited for here, visibly to the compiler, so that it places no wait for
      // them inside the loop (where it would also drain the tile copies).
      if (pass == 0 && spec_ok) {
        wait_vmem_lds<0>();                     // the speculative copies were right
      } else {
        wait_vmem_lds<0>();                     // speculative copies land before their buffers are reused
        stage(0, lds_addr(s_tiles[0]));
        if (n_tiles > 1) stage(1, lds_addr(s_tiles[1]));
        else stage_rows(0, lds_addr(s_tiles[1]), 1);
      }
#pragma unroll
      for (int k = 2; k < NBUF - 1; ++k) {
        if (k < n_tiles) stage(k, lds_addr(s_tiles[k]));
        else stage_rows(0, lds_addr(s_tiles[k]), 1);
      }
#pragma unroll 1
      for (int tile = 0; tile < n_tiles; tile += NBUF) {
#pragma unroll
        for (int k = 0; k < NBUF; ++k) {
          const int t = tile + k;
          if (t >= n_tiles) break;
          wait_tile();
          const bool real = t + NBUF - 1 < n_tiles;
          const int st = real ? t + NBUF - 1 : t;
          const int st_rows = real ? min(kBN, k_end - (k_begin + st * kBN)) : 1;
          const uint32_t sb = lds_addr(s_tiles[(k + NBUF - 1) % NBUF]);
          if (compute) tile_body(t, s_tiles[k], st, st_rows, sb);
          else stage_rows(st, sb, st_rows);
        }
      }
      wait_vmem_lds<0>();                       // the last (dummy) copies land before anything else
    }

    // Key streams: the two waves of a row block share the output, stream s
    // writing column half s.  Each leaves the other half of its accumulators,
    // its reference and its sum in the (now idle) tile ring for its partner,
    // then rescales both streams to the larger reference as it writes its half
    // (the partner's accumulators are read block by block in the loops below).
    constexpr int XS = (NBL / 2 * 16 + 2) * 64; // floats per wave
    float* xw = reinterpret_cast<float*>(&s_tiles[0][0]) + wave * XS;
    const float* xr = reinterpret_cast<const float*>(&s_tiles[0][0]) + (wave ^ 1) * XS;
    float f0 = 1.0f, f1 = 0.0f;
    if constexpr (KS) {
      tile_barrier();                           // every wave is done with the ring
#pragma unroll
      for (int db = NBL / 2; db < NBL; ++db) {  // (blocks 0-7 are the half this wave keeps)
        // straight from the accumulation registers; the four groups of block
        // db sit 1 KB apart, each lane's 16 bytes consecutive across lanes
        const uint32_t ad = lds_addr(xw + (((db & 7) * 4) * 64 + lane) * 4);
        asm volatile(
            "ds_write_b128 %0, %1\n\t"
            "ds_write_b128 %0, %2 offset:1024\n\t"
            "ds_write_b128 %0, %3 offset:2048\n\t"
            "ds_write_b128 %0, %4 offset:3072"
            :
            : "v"(ad), "a"(__builtin_shufflevector(acc[db], acc[db], 0, 1, 2, 3)),
              "a"(__builtin_shufflevector(acc[db], acc[db], 4, 5, 6, 7)),
              "a"(__builtin_shufflevector(acc[db], acc[db], 8, 9, 10, 11)),
              "a"(__builtin_shufflevector(acc[db], acc[db], 12, 13, 14, 15))
            : "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
      xw[NBL / 2 * 16 * 64 + lane] = m_ref;
      xw[NBL / 2 * 16 * 64 + 64 + lane] = l_run;
      wait_lds();                               // (also the asm stores above)
      tile_barrier();
      const float m1 = xr[NBL / 2 * 16 * 64 + lane], l1 = xr[NBL / 2 * 16 * 64 + 64 + lane];
      const float mt = fmaxf(m_ref, m1);
      f0 = m_ref == -INFINITY ? 0.0f : exp2f(m_ref - mt);
      f1 = m1 == -INFINITY ? 0.0f : exp2f(m1 - mt);
      l_run = l_run * f0 + l1 * f1;
      m_ref = mt;
    }
    // the accumulator blocks this wave writes (key streams: blocks 0-7, its
    // column half)
    auto own_block = [&](int db) { return !KS || db < NBL / 2; };
    // ---- epilogue: normalise and write (direct) or write the partial
    const float l_tot = xhalf_sum(l_run);
    const float m_fin = (m_ref == -INFINITY) ? 0.0f : m_ref;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float lse_v = l_tot > 0.0f ? (m_fin + log2f(l_tot)) * kLn2 : -INFINITY;
    // key streams: the normalisation folded into the two streams' factors
    f0 *= inv;
    f1 *= inv;
    // normalised output (db, 4 g + e) of this lane, both key streams combined
    auto out_of = [&](int db, int g, f32x4& v) __attribute__((always_inline)) {
      if constexpr (KS) {
        // the partner's accumulator block db + 8 (the same output columns)
        const f32x4 o = *reinterpret_cast<const f32x4*>(xr + (((db & 7) * 4 + g) * 64 + lane) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[db][4 * g + e] * f0 + o[e] * f1;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[db][4 * g + e] * inv;
      }
    };
    // a sequence with one split needs no merge: the fused launch writes its
    // output directly too
    const int ns_b = sr.ns;
    const bool direct_now = DIRECT || (a.fuse && ns_b == 1);
    if (direct_now) {
      if (row_ok) {
        T* o = reinterpret_cast<T*>(a.out) + b * a.out_sb + t * a.out_st + h * a.out_sh;
#pragma unroll
        for (int db = 0; db < NBL; ++db) {
          if (!own_block(db)) continue;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 av;
            out_of(db, g, av);
            const float v4[4] = {av[0], av[1], av[2], av[3]};
            store4<T>(o + col_block(db) * 32 + 8 * g + 4 * hh, v4);
          }
          if constexpr (KS) __builtin_amdgcn_sched_barrier(0);   // one block's partner values at a time
        }
        if (hh == 0 && chalf == 0 && kp == 0) a.lse[(int64_t)b * a.M + m] = lse_v;
      }
    } else if (!DIRECT) {
      if (row_ok) {
        // Partials stay in accumulator order: the wave's 32 rows form one block
        // of 32 x R values in which every store instruction writes one contiguous
        // 1 KB run (float32: register group (db, g) of every lane; bf16: groups
        // (db, 2p) and (db, 2p + 1) packed into 16 bytes per lane).  Streaming,
        // device-coherent stores: the merge reads them from other compute units.
        const int blk = rt * (BM / 32) + rb;
        const int64_t base = (((int64_t)b * a.max_splits + split) * a.n_blk + blk) * (32 * R);
        if (a.part_bf16) {
          __bf16* o = static_cast<__bf16*>(a.part_o) + base;
#pragma unroll
          for (int db = 0; db < NBL; ++db) {
            if (!own_block(db)) continue;
#pragma unroll
            for (int gp = 0; gp < 2; ++gp) {
              f32x4 a0, a1;
              out_of(db, 2 * gp, a0);
              out_of(db, 2 * gp + 1, a1);
              bf16x8 v8;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                v8[e] = (__bf16)a0[e];
                v8[4 + e] = (__bf16)a1[e];
              }
              store16_coherent(o, (uint32_t)(16 * lane + 1024 * (2 * col_block(db) + gp)), v8);
            }
            if constexpr (KS) __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          float* o = static_cast<float*>(a.part_o) + base;
#pragma unroll
          for (int db = 0; db < NBL; ++db) {
            if (!own_block(db)) continue;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              f32x4 av;
              out_of(db, g, av);
              store16_coherent(o, (uint32_t)(16 * lane + 1024 * (4 * col_block(db) + g)), av);
            }
            if constexpr (KS) __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      if (row_ok && hh == 0 && chalf == 0 && kp == 0)
        __hip_atomic_store(a.part_lse + ((int64_t)b * a.max_splits + split) * a.M + m, lse_v, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      if (a.fuse) {
        fused_merge<T, R>(a, b, rt, split, ns_b, BM, reinterpret_cast<float*>(&s_tiles[0][0]), tid);
      }
    }
  }  // pieces
}

// WIDE: one (sequence, block, column group) per workgroup; used when there
// are more splits than one wave loads in one round trip.  Otherwise one item
// per wave.
template <typename T, typename PT, bool WIDE, bool GATE, int U>
__global__ __launch_bounds__(256) void merge_kernel(
    const PT* __restrict__ part_o, const float* __restrict__ part_lse, int max_splits,
    int B, int q, int H, int R, int n_blk, const int32_t* __restrict__ prefix_lens, int split_keys, int tiles_max,
    T* __restrict__ out, int64_t out_sb, int64_t out_st, int64_t out_sh, float* __restrict__ lse) {
  constexpr int NV = PartLoad<PT>::NV;
  __shared__ float s_st[WIDE ? 4 * (NV + 2) * 64 : 1];
  const int n_cg = R / (2 * NV);
  const int wave = threadIdx.x >> 6;
  // (the host keeps the item count under 2^31, so the item index and its
  // decomposition are 32-bit: 64-bit divisions would put a few hundred scalar
  // instructions before the first load)
  const uint32_t wid = WIDE ? blockIdx.x : blockIdx.x * (blockDim.x >> 6) + (uint32_t)wave;
  const int lane = threadIdx.x & 63;
  if (wid >= (uint32_t)B * (uint32_t)n_blk * (uint32_t)n_cg) return;  // (uniform over the workgroup when WIDE)
  const int cg = (int)(wid % (uint32_t)n_cg);
  const uint32_t bblk = wid / (uint32_t)n_cg;
  const int blk = (int)(bblk % (uint32_t)n_blk), b = (int)(bblk / (uint32_t)n_blk);
  const int M = q * H;
  int ns = max_splits;
  if (split_keys > 0) {
    const int L = prefix_lens[b];
    // (a skipped sequence wrote empty partials: any count is right)
    ns = L >= 0 && L <= 0x7FFFFFFF - q ? split_range(L + q, 0, split_keys, max_splits, tiles_max).ns : max_splits;
  }
  merge_item<T, PT, WIDE, false, GATE, U>(part_o, part_lse, max_splits, ns, M, H, R, n_blk, b, blk, cg, out, out_sb,
                                       out_st, out_sh, lse, s_st, wave, lane);
}

// ---------------------------------------------------------------------------
// Host side

static int elem_size(int dtype) { return dtype == KDT_F32 ? 4 : dtype == KDT_BF16 ? 2 : 0; }

// Compute units of the current device (host query, cached per device; kCU
// when the runtime cannot say).
static int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kCU;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = kCU;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

constexpr int kDefaultWaitUs = 2000;     // longest wait of a split workgroup in the fused merge

static bool shape_supported(int dtype, int R, int P) {
  if (dtype == KDT_BF16) return (R == 512 && P == 64) || (R == 64 && P == 16);
  if (dtype == KDT_F32) return R == 64 && P == 16;
  return false;
}

// Layouts 3 (depth-split score pairs) and 4 (two key streams) are built for
// the bf16 rank-512 shape.
static bool wide_layout_supported(int dtype, int R, int P) { return dtype == KDT_BF16 && R == 512 && P == 64; }

static int validate(const kdt_verify_desc* d) {
  if (!d) return KDT_ERR_INVALID_ARG;
  if (d->B <= 0 || d->q_len <= 0 || d->H <= 0 || d->R <= 0 || d->P <= 0) return KDT_ERR_INVALID_ARG;
  if (!d->q_lat || !d->q_pe || !d->c_kv || !d->k_pe || !d->prefix_lens || (!d->vis && !d->parents) || !d->out ||
      !d->lse)
    return KDT_ERR_INVALID_ARG;
  if (d->max_prefix_len < 0 || d->capacity < (int64_t)d->max_prefix_len + d->q_len)
    return KDT_ERR_INVALID_ARG;
  if (d->split_keys < 0 || (d->split_keys % kBN) != 0) return KDT_ERR_INVALID_ARG;
  if (d->layout < 0 || d->layout > 4) return KDT_ERR_INVALID_ARG;
  if (d->partials_f32 != 0 && d->partials_f32 != 1) return KDT_ERR_INVALID_ARG;
  if (d->merge_mode != 0 && d->merge_mode != 1) return KDT_ERR_INVALID_ARG;
  if (d->schedule < 0 || d->schedule > 2 || d->gang_size < 0) return KDT_ERR_INVALID_ARG;
  if (d->schedule == 2 && d->split_keys != 0) return KDT_ERR_INVALID_ARG;
  if ((int64_t)d->max_prefix_len + d->q_len > 0x7FFFFFFF - kBN) return KDT_ERR_UNSUPPORTED;
  if (!(d->softmax_scale > 0.0f) || !isfinite(d->softmax_scale)) return KDT_ERR_INVALID_ARG;
  if (d->q_len > KDT_MAX_Q_LEN) return KDT_ERR_UNSUPPORTED;
  if (!shape_supported(d->dtype, d->R, d->P)) return KDT_ERR_UNSUPPORTED;
  const int64_t vec = 16 / elem_size(d->dtype);   // elements per 16 bytes
  if (!aligned16(d->q_lat) || !aligned16(d->q_pe) || !aligned16(d->c_kv) || !aligned16(d->k_pe) ||
      !aligned16(d->out))
    return KDT_ERR_UNSUPPORTED;
  const int64_t strides[] = {d->q_lat_sb, d->q_lat_st, d->q_lat_sh, d->q_pe_sb, d->q_pe_st, d->q_pe_sh,
                             d->c_kv_sb, d->c_kv_ss, d->k_pe_sb, d->k_pe_ss,
                             d->out_sb, d->out_st, d->out_sh};
  for (int64_t s : strides)
    if (s < 0 || s % vec) return KDT_ERR_UNSUPPORTED;
  if ((int64_t)d->B * d->q_len * d->H > 0x7FFFFFFF) return KDT_ERR_UNSUPPORTED;
  if (d->layout >= 3 && !wide_layout_supported(d->dtype, d->R, d->P)) return KDT_ERR_UNSUPPORTED;
  return KDT_OK;
}

// Rows per workgroup of a layout (1: four waves x 32 rows; 2: two row blocks,
// each shared by a wave pair that splits the output columns).
static int layout_rows(int layout) { return layout >= 2 ? kBM / 2 : kBM; }

// Modelled time (microseconds) of one launch, split kernel plus merge, for a
// layout, split size and count: `wgs` split workgroups with work (one per
// compute unit, so ceil(wgs / kCU) rounds) of at most `tiles` key tiles each;
// a round costs its tiles plus a start-up (the burst of query and first-tile
// loads), every partial costs its write and its read in the merge, and
// splitting at all adds the merge launch plus one memory round trip per
// batch of splits the merge loads at once (sixteen per wave; up to sixty-four
// when a workgroup's four waves share the splits of one item).  The constants
// are fitted to a measured grid of split sizes and layouts over six workloads
// at R = 512, P = 64 (a 128-row tile of 32 keys about 1.7 us, a start-up about
// 4 us) and scale with the contraction work of one wave and with the bytes a
// partial holds.  The partial's cost, 0.10 us for 128 float32 rows, was
// refitted once partials were bf16 and the loop faster: at max_budget 14
// splits of 320 keys then beat 11 of 384 (step 34.7 against 35.5 us).
static double launch_cost(int64_t wgs, int64_t splits, int64_t tiles, int R, int P, int layout, int part_bytes) {
  const int rows = layout_rows(layout);
  // layout 4: two key tiles per step, each wave doing layout 1's work for its
  // tile in about 1.1 times layout 1's tile time, plus about 2 us to combine
  // the two streams at the end
  const double t_tile = layout == 4 ? 1.7 * 1.1 / 2.0 : 1.7 * ((double)R + P + (double)R * rows / kBM) / (2.0 * R + P);
  const double t_start = layout == 4 ? 6.0 : 4.0;
  const double t_part = 0.10 * rows / kBM * R / 512.0 * part_bytes / 4.0;
  const double t_merge = 3.0, t_merge_batch = 2.0;
  const int64_t rounds = (wgs + kCU - 1) / kCU;
  const int64_t batches = splits > 16 ? (splits + 63) / 64 : 1;
  const double merge = splits > 1 ? wgs * t_part + t_merge + t_merge_batch * (double)batches : 0.0;
  // (layout 4 works in steps of two tiles: an odd tile count wastes half a step)
  const int64_t t = layout == 4 ? (tiles + 1) / 2 * 2 : tiles;
  return rounds * (t * t_tile + t_start) + merge;
}

// Modelled time of the balanced schedule: one round, every gang doing A key
// tiles in `pieces` pieces, each paying a start-up, plus the merge of `parts`
// partial row tiles of `splits` slots (gated loads: one more round trip), plus
// a share of the time the cache takes to stream `reads` times past the compute
// units (each row-tile group reads every key once; the members of a gang share
// one read through their XCD's L2; measured: gangs of one row tile, every
// workgroup reading its keys alone, ran 6-8% slower than gangs of 5 to 11).
// Same constants as launch_cost otherwise.
static double tile_time(int R, int P, int layout) {
  const int rows = layout_rows(layout);
  return layout == 4 ? 1.7 * 1.1 / 2.0 : 1.7 * ((double)R + P + (double)R * rows / kBM) / (2.0 * R + P);
}

// Balanced schedule: the start-up and epilogue of a piece (measured 10-11 us
// in a full launch: the query loads of every workgroup at once dominate) in
// key tiles; every stream is charged this many units before its key tiles.
constexpr double kPieceUs = 10.0;
static int piece_units(int R, int P, int layout) { return (int)std::ceil(kPieceUs / tile_time(R, P, layout)); }

static double balanced_cost(int64_t A, double pieces, int64_t parts, int64_t splits, int64_t reads,
                            double cache_bytes, int R, int P, int layout, int part_bytes) {
  const int rows = layout_rows(layout);
  const double t_tile = tile_time(R, P, layout);
  const double t_start = layout == 4 ? 6.0 : 4.0;
  const double t_part = 0.10 * rows / kBM * R / 512.0 * part_bytes / 4.0;
  const double t_merge = 3.0, t_merge_batch = 2.0;
  const int64_t batches = splits > 16 ? (splits + 63) / 64 : 1;
  const double t_fetch = 0.15 * (double)reads * cache_bytes / 8.0e6;   // us at 8 TB/s
  return A * t_tile + pieces * t_start + parts * t_part + t_merge + t_merge_batch * (double)(batches + 1) + t_fetch;
}

constexpr int kBalancedMaxB = 4096;      // the walk scans the prefix lengths in every workgroup

static int make_plan(const kdt_verify_desc* d, kdt_verify_plan* p) {
  const int rc = validate(d);
  if (rc != KDT_OK) return rc;
  const int M = d->q_len * d->H;
  const int64_t n_max = (int64_t)d->max_prefix_len + d->q_len;
  const int64_t tiles_max = (n_max + kBN - 1) / kBN;
  const int part_dtype = (d->dtype == KDT_BF16 && !d->partials_f32) ? KDT_BF16 : KDT_F32;
  // The split kernel addresses a split's cache rows by 32-bit byte offsets
  // from its first row: split_keys rows of either region stay under 2^31 bytes.
  const int64_t row_bytes = (d->c_kv_ss > d->k_pe_ss ? d->c_kv_ss : d->k_pe_ss) * elem_size(d->dtype);
  const int64_t max_sk = row_bytes > 0 ? 0x7FFFFFFF / row_bytes / kBN * kBN : (int64_t)1 << 40;
  if (max_sk < kBN || d->split_keys > max_sk) return KDT_ERR_UNSUPPORTED;
  // Key tiles of all sequences together: from the caller's hint (the sum of
  // the prefix lengths), else as if every sequence had the longest length.
  const int64_t total_keys = d->total_prefix_len > 0 ? d->total_prefix_len + (int64_t)d->B * d->q_len
                                                     : (int64_t)d->B * n_max;
  const int64_t total_tiles = (total_keys + kBN - 1) / kBN + d->B / 2;
  // With the library's choice of split size the splits are adaptive: every
  // sequence is cut into splits of about the same number of tiles as the
  // longest one's (split_range), so the split workgroups with work number
  // about s * total_tiles / tiles_max (each sequence rounding up), not B * s.
  const bool adaptive = d->split_keys == 0;
  int best_layout = d->layout ? d->layout : 1;
  int64_t sk = d->split_keys;
  double best = 1e300;
  const bool wide_ok = wide_layout_supported(d->dtype, d->R, d->P);
  for (int layout = 1; layout <= 4; ++layout) {
    if (d->layout ? layout != d->layout : (layout == 3 || (layout == 4 && !wide_ok))) continue;
    const int64_t n_rt = (M + layout_rows(layout) - 1) / layout_rows(layout);
    for (int64_t s = 1; s <= tiles_max && s <= 4096; ++s) {
      int64_t k;
      if (d->split_keys) {
        k = d->split_keys;
      } else {
        const int64_t tps = (tiles_max + s - 1) / s;
        if ((tiles_max + tps - 1) / tps != s) continue;      // covered by a smaller s
        k = tps * kBN;
      }
      if (k > max_sk) continue;
      const int64_t ns = (n_max + k - 1) / k;
      // (each sequence rounds its own split count up: half a split on average)
      const int64_t per_seq = adaptive ? (ns * total_tiles + tiles_max - 1) / tiles_max + (d->B + 1) / 2
                                       : (total_keys + k - 1) / k + (d->B + 1) / 2;
      const int64_t wgs = n_rt * std::min((int64_t)d->B * ns, std::max<int64_t>(per_seq, 1));
      const double c = launch_cost(wgs, ns, k / kBN, d->R, d->P, layout, elem_size(part_dtype));
      if (c < best * 0.999) {                 // ties go to fewer splits, then layout 1
        best = c;
        sk = k;
        best_layout = layout;
      }
      if (d->split_keys) break;
    }
  }
  // The balanced schedule: every layout and gang size, one round of
  // workgroups.  Chosen over splits only where the model says it is faster
  // (the fused merge, on request, needs splits).
  int64_t bal_g = 0, bal_G = 0, bal_S = 0, bal_A = 0;
  const bool bal_ok = d->split_keys == 0 && d->schedule != 1 && d->B <= kBalancedMaxB &&
                      (d->schedule == 2 || d->merge_mode == 0);
  if (bal_ok) {
    const int cus = device_cus();
    const int64_t lim = max_sk / kBN;            // key tiles one piece may span
    double bal_best = d->schedule == 2 ? 1e300 : best;
    for (int layout = 1; layout <= 2; ++layout) {
      if (d->layout && layout != d->layout) continue;
      const int64_t n_rt = (M + layout_rows(layout) - 1) / layout_rows(layout);
      for (int64_t g = 1; g <= n_rt && g <= cus; ++g) {
        if (d->gang_size && g != d->gang_size) continue;
        const int64_t G = cus / g;
        const int64_t n_grp = (n_rt + g - 1) / g;
        const int64_t U = n_grp * (total_tiles + (int64_t)d->B * piece_units(d->R, d->P, layout));
        // (the walk counts units in 32 bits: every sequence at its longest must fit)
        if ((double)n_grp * d->B * (double)(tiles_max + piece_units(d->R, d->P, layout)) > 2.0e9) continue;
        const int64_t A = std::min(lim, std::max<int64_t>(1, (U + G - 1) / G));
        const int64_t S = std::max<int64_t>({2, (tiles_max + A - 1) / A + 1, (tiles_max + lim - 1) / lim + 1});
        const int64_t streams = (int64_t)d->B * n_grp;
        const double pieces = 1.0;              // (later pieces' start-ups are inside A)
        const int64_t parts = std::min(G + streams, streams * S) * g;
        const double kv_bytes = (double)total_keys * (double)(d->R + d->P) * elem_size(d->dtype);
        const double c = balanced_cost(A, pieces, parts, S, n_grp, kv_bytes, d->R, d->P, layout,
                                       elem_size(part_dtype)) *
                         (double)((U + G - 1) / G > lim ? ((U + G - 1) / G + lim - 1) / lim : 1);
        if (c < bal_best * 0.999) {
          bal_best = c;
          bal_g = g;
          bal_G = G;
          bal_S = S;
          bal_A = A;
          best_layout = layout;
        }
      }
    }
    // (on request: layouts 1 and 2 only, a gang no larger than the row tiles,
    // and lengths the walk can count in 32 bits)
    if (d->schedule == 2 && !bal_g) {
      const bool too_long = (double)d->B * (double)(tiles_max + piece_units(d->R, d->P, 1)) > 2.0e9;
      return d->layout > 2 || too_long ? KDT_ERR_UNSUPPORTED : KDT_ERR_INVALID_ARG;
    }
  }
  p->layout = best_layout;
  p->part_dtype = part_dtype;
  p->gang_size = (int32_t)bal_g;
  p->gangs = (int32_t)bal_G;
  p->piece_units = bal_g ? piece_units(d->R, d->P, best_layout) : 0;
  if (bal_g) sk = bal_A * kBN;
  if (sk <= 0) return KDT_ERR_UNSUPPORTED;   // no split size fits the row offsets
  const int64_t ns = bal_g ? bal_S : (n_max + sk - 1) / sk;
  if (ns > 0x7FFFFFFF / 2) return KDT_ERR_UNSUPPORTED;
  p->split_keys = (int32_t)(sk > 0x7FFFFFFF ? 0x7FFFFFFF : sk);
  p->max_splits = (int32_t)ns;
  p->tiles_max = adaptive && ns > 1 && !bal_g ? (int32_t)tiles_max : 0;
  p->rows = M;
  p->direct = ns == 1 && !bal_g ? 1 : 0;
  const int64_t n_part_rows = (int64_t)d->B * ns * M;
  const int64_t o_bytes = (int64_t)d->B * ns * ((M + 31) / 32) * 32 * d->R * elem_size(part_dtype);
  p->part_o_offset = 0;
  p->part_lse_offset = (o_bytes + 255) / 256 * 256;
  p->partials_bytes = (size_t)(p->part_lse_offset + n_part_rows * 4);
  // merge inside the split kernel on request, when every split workgroup can
  // be resident at once (one workgroup per compute unit)
  const int64_t n_rt = (M + layout_rows(p->layout) - 1) / layout_rows(p->layout);
  const int64_t grid = (int64_t)d->B * n_rt * ns;
  p->fused_merge = (!p->direct && !bal_g && d->merge_mode == 1 && grid <= device_cus()) ? 1 : 0;
  p->counter_offset = ((int64_t)p->partials_bytes + 255) / 256 * 256;
  p->workspace_bytes = p->direct ? 0 : (size_t)(p->counter_offset + (int64_t)d->B * n_rt * 4);
  return KDT_OK;
}

// A stride near 0.618 of n (the golden ratio spreads the multiples evenly)
// that is coprime to n, so g -> g * stride mod n is a permutation of 0 .. n-1.
static int group_stride(int64_t n) {
  if (n <= 2) return 1;
  int64_t m = (int64_t)((double)n * 0.6180339887498949);
  if (m < 1) m = 1;
  auto gcd = [](int64_t x, int64_t y) {
    while (y) {
      const int64_t t = x % y;
      x = y;
      y = t;
    }
    return x;
  };
  while (gcd(m, n) != 1) ++m;
  return (int)m;
}

static VerifyArgs make_args(const kdt_verify_desc* d, const kdt_verify_plan& p, void* ws, bool fuse) {
  VerifyArgs a;
  a.fuse = fuse ? 1 : 0;
  a.counters = (ws && fuse) ? reinterpret_cast<int32_t*>(static_cast<char*>(ws) + p.counter_offset) : nullptr;
  const int64_t wait_us = d->merge_wait_us == 0 ? kDefaultWaitUs : (d->merge_wait_us < 0 ? 0 : d->merge_wait_us);
  a.spin_ticks = wait_us * 100;          // 100 MHz
  a.q_lat = d->q_lat; a.q_lat_sb = d->q_lat_sb; a.q_lat_st = d->q_lat_st; a.q_lat_sh = d->q_lat_sh;
  a.q_pe = d->q_pe; a.q_pe_sb = d->q_pe_sb; a.q_pe_st = d->q_pe_st; a.q_pe_sh = d->q_pe_sh;
  a.c_kv = d->c_kv; a.c_kv_sb = d->c_kv_sb; a.c_kv_ss = d->c_kv_ss;
  a.k_pe = d->k_pe; a.k_pe_sb = d->k_pe_sb; a.k_pe_ss = d->k_pe_ss;
  a.capacity = d->capacity;
  a.prefix_lens = d->prefix_lens;
  a.vis = d->vis;
  a.parents = d->vis ? nullptr : d->parents;
  a.out = d->out; a.out_sb = d->out_sb; a.out_st = d->out_st; a.out_sh = d->out_sh;
  a.lse = d->lse;
  a.part_o = ws ? static_cast<void*>(static_cast<char*>(ws) + p.part_o_offset) : nullptr;
  a.part_bf16 = p.part_dtype == KDT_BF16;
  a.part_lse = ws ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.part_lse_offset) : nullptr;
  a.seq_status = d->seq_status;
  a.scale_log2 = d->softmax_scale * kLog2e;
  a.B = d->B; a.q = d->q_len; a.H = d->H; a.M = d->q_len * d->H; a.W = (d->q_len + 63) / 64;
  a.layout = p.layout;
  a.n_rt = (a.M + layout_rows(p.layout) - 1) / layout_rows(p.layout);
  a.n_blk = (a.M + 31) / 32;
  a.max_splits = p.max_splits;
  a.split_keys = p.split_keys;
  a.tiles_max = p.tiles_max;
  a.group_mul = group_stride((int64_t)d->B * p.max_splits);
  a.compact = p.tiles_max > 0 && d->B > 1;
  a.gang = p.gang_size;
  a.gangs = p.gangs;
  a.piece_units = p.piece_units;
  a.n_grp = p.gang_size > 0 ? (a.n_rt + p.gang_size - 1) / p.gang_size : 0;
  {
    // a piece's cache rows of either region stay under 2^31 bytes from its first
    const int64_t row_bytes = std::max(d->c_kv_ss, d->k_pe_ss) * elem_size(d->dtype);
    const int64_t max_sk = row_bytes > 0 ? 0x7FFFFFFF / row_bytes / kBN * kBN : 0x7FFFFFE0;
    a.span_keys = p.gang_size > 0 ? (int)std::min<int64_t>(max_sk, 0x7FFFFFE0) : p.split_keys;
  }
  a.max_prefix_len = d->max_prefix_len;
  const int64_t es = elem_size(d->dtype);
  a.q_rows_uniform = d->q_lat_st == (int64_t)d->H * d->q_lat_sh && d->q_pe_st == (int64_t)d->H * d->q_pe_sh &&
                     d->q_lat_sh * es < (1ll << 26) && d->q_pe_sh * es < (1ll << 26);
  return a;
}

template <typename T, int R, int P>
static int launch_split(const VerifyArgs& a, bool direct, hipStream_t s) {
  const int64_t grid = a.gang ? (int64_t)a.gangs * a.gang : (int64_t)a.B * a.n_rt * a.max_splits;
  if (grid > 0x7FFFFFFF) return KDT_ERR_UNSUPPORTED;
  const bool cs2 = a.layout == 2;
  if (a.gang) {
    if (direct || (a.layout != 1 && a.layout != 2)) return KDT_ERR_UNSUPPORTED;
    if (cs2)
      hipLaunchKernelGGL((verify_split_kernel<T, R, P, false, 2, true>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((verify_split_kernel<T, R, P, false, 1, true>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
    return launch_status();
  }
  if constexpr (R == 512 && P == 64 && sizeof(T) == 2) {
    if (a.layout == 3) {
      if (direct)
        hipLaunchKernelGGL((verify_split_kernel<T, R, P, true, 3>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
      else
        hipLaunchKernelGGL((verify_split_kernel<T, R, P, false, 3>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
      return launch_status();
    }
    if (a.layout == 4) {
      if (direct)
        hipLaunchKernelGGL((verify_split_kernel<T, R, P, true, 4>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
      else
        hipLaunchKernelGGL((verify_split_kernel<T, R, P, false, 4>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
      return launch_status();
    }
  }
  if (direct && cs2)
    hipLaunchKernelGGL((verify_split_kernel<T, R, P, true, 2>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else if (direct)
    hipLaunchKernelGGL((verify_split_kernel<T, R, P, true, 1>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else if (cs2)
    hipLaunchKernelGGL((verify_split_kernel<T, R, P, false, 2>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((verify_split_kernel<T, R, P, false, 1>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return launch_status();
}

static int dispatch_split(int dtype, int R, int P, const VerifyArgs& a, bool direct, hipStream_t s) {
  if (dtype == KDT_BF16 && R == 512 && P == 64) return launch_split<__bf16, 512, 64>(a, direct, s);
  if (dtype == KDT_BF16 && R == 64 && P == 16) return launch_split<__bf16, 64, 16>(a, direct, s);
  if (dtype == KDT_F32 && R == 64 && P == 16) return launch_split<float, 64, 16>(a, direct, s);
  return KDT_ERR_UNSUPPORTED;
}

template <typename PT>
static int launch_merge_t(int dtype, int B, int q, int H, int R, const PT* po, const float* pl, int max_splits,
                          const int32_t* prefix_lens, int split_keys, int tiles_max, bool gate, void* out,
                          int64_t osb, int64_t ost, int64_t osh, float* lse, hipStream_t s) {
  const int n_blk = (q * H + 31) / 32;
  const int64_t items = (int64_t)B * n_blk * (R / (2 * PartLoad<PT>::NV));
  // more splits than one wave loads in one round trip: a workgroup per item
  const bool wide = max_splits > 16;
  const int64_t grid = wide ? items : (items + 3) / 4;
  if (items > 0x7FFFFFFF) return KDT_ERR_UNSUPPORTED;
  // splits per round trip: the fewest of 4, 8 and 16 that hold every split
  // (the sums then run in the same order whatever the choice)
  const int u = wide ? 16 : (max_splits <= 4 ? 4 : (max_splits <= 8 ? 8 : 16));
#define KDT_MERGE_LAUNCH(TO, W, GT, UU)                                                                      \
  hipLaunchKernelGGL((merge_kernel<TO, PT, W, GT, UU>), dim3((unsigned)grid), dim3(256), 0, s, po, pl, max_splits, \
                     B, q, H, R, n_blk, prefix_lens, split_keys, tiles_max, static_cast<TO*>(out), osb, ost, osh, lse)
#define KDT_MERGE_U(TO, GT)                                 \
  do {                                                      \
    if (wide) KDT_MERGE_LAUNCH(TO, true, GT, 16);           \
    else if (u == 4) KDT_MERGE_LAUNCH(TO, false, GT, 4);    \
    else if (u == 8) KDT_MERGE_LAUNCH(TO, false, GT, 8);    \
    else KDT_MERGE_LAUNCH(TO, false, GT, 16);               \
  } while (0)
  if (dtype == KDT_BF16) {
    if (gate) KDT_MERGE_U(__bf16, true);
    else KDT_MERGE_U(__bf16, false);
  } else {
    if (gate) KDT_MERGE_U(float, true);
    else KDT_MERGE_U(float, false);
  }
#undef KDT_MERGE_U
#undef KDT_MERGE_LAUNCH
  return launch_status();
}

static int launch_merge(int dtype, int B, int q, int H, int R, int part_dtype, const void* po, const float* pl,
                        int max_splits, const int32_t* prefix_lens, int split_keys, int tiles_max, bool gate,
                        void* out, int64_t osb, int64_t ost, int64_t osh, float* lse, hipStream_t s) {
  if (part_dtype == KDT_BF16)
    return launch_merge_t(dtype, B, q, H, R, static_cast<const __bf16*>(po), pl, max_splits, prefix_lens,
                          split_keys, tiles_max, gate, out, osb, ost, osh, lse, s);
  return launch_merge_t(dtype, B, q, H, R, static_cast<const float*>(po), pl, max_splits, prefix_lens, split_keys,
                        tiles_max, gate, out, osb, ost, osh, lse, s);
}

// The verify with a given workspace (NULL when the plan is direct).
static int verify_run(const kdt_verify_desc* d, const kdt_verify_plan& p, void* workspace, hipStream_t s) {
  const VerifyArgs a = make_args(d, p, p.direct ? nullptr : workspace, p.fused_merge != 0);
  int r = dispatch_split(d->dtype, d->R, d->P, a, p.direct != 0, s);
  if (r != KDT_OK || p.direct || p.fused_merge) return r;
  // (balanced schedule: every slot of a row is merged, the empty ones skipped
  // by their log-sum-exp)
  const bool bal = p.gang_size > 0;
  return launch_merge(d->dtype, d->B, d->q_len, d->H, d->R, p.part_dtype, a.part_o, a.part_lse, p.max_splits,
                      d->prefix_lens, bal ? 0 : p.split_keys, bal ? 0 : p.tiles_max, bal, d->out, d->out_sb,
                      d->out_st, d->out_sh, d->lse, s);
}

// Workspace of kdt_verify_attn_noalloc: a fixed device array, one per GPU
// (each device that loads the library holds its own copy until the process
// ends).  Host code never uses the array's name as an address: the device
// address of each GPU's copy is looked up once, with that GPU current, and
// kept.
constexpr size_t kScratchBytes = KDT_NOALLOC_MAX_WORKSPACE;
__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;

static void* scratch_ptr() {
  static std::mutex mu;
  static void* ptrs[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

}  // namespace kdt

extern "C" int kdt_verify_get_plan(const kdt_verify_desc* d, kdt_verify_plan* plan) {
  if (!plan) return KDT_ERR_INVALID_ARG;
  return kdt::make_plan(d, plan);
}

extern "C" int kdt_verify_attn(const kdt_verify_desc* d, void* workspace, size_t ws_bytes, void* stream) {
  kdt_verify_plan p;
  const int rc = kdt::make_plan(d, &p);
  if (rc != KDT_OK) return rc;
  if (!p.direct && (!workspace || ws_bytes < p.workspace_bytes)) return KDT_ERR_WORKSPACE;
  if (!p.direct && !kdt::aligned16(workspace)) return KDT_ERR_WORKSPACE;
  return kdt::verify_run(d, p, workspace, static_cast<hipStream_t>(stream));
}

extern "C" int kdt_verify_attn_noalloc(const kdt_verify_desc* d, void* stream) {
  kdt_verify_plan p;
  const int rc = kdt::make_plan(d, &p);
  if (rc != KDT_OK) return rc;
  // the merge state words of the in-kernel merge would have to start at zero
  if (d->merge_mode != 0) return KDT_ERR_UNSUPPORTED;
  if (p.workspace_bytes > kdt::kScratchBytes) return KDT_ERR_WORKSPACE;
  void* ws = nullptr;
  if (!p.direct) {
    ws = kdt::scratch_ptr();
    if (!ws) return KDT_ERR_LAUNCH;
  }
  return kdt::verify_run(d, p, ws, static_cast<hipStream_t>(stream));
}

extern "C" int kdt_verify_partials(const kdt_verify_desc* d, void* workspace, size_t ws_bytes,
                                   void* stream) {
  kdt_verify_plan p;
  const int rc = kdt::make_plan(d, &p);
  if (rc != KDT_OK) return rc;
  if (!workspace || ws_bytes < p.partials_bytes || !kdt::aligned16(workspace)) return KDT_ERR_WORKSPACE;
  const kdt::VerifyArgs a = kdt::make_args(d, p, workspace, false);
  return kdt::dispatch_split(d->dtype, d->R, d->P, a, false, static_cast<hipStream_t>(stream));
}

extern "C" int kdt_merge_partials(int32_t dtype, int32_t B, int32_t q_len, int32_t H, int32_t R,
                                  int32_t part_dtype, const void* part_o, const float* part_lse, int32_t max_splits,
                                  const int32_t* prefix_lens, int32_t split_keys, void* out,
                                  int64_t out_sb, int64_t out_st, int64_t out_sh, float* lse,
                                  void* stream) {
  if (!part_o || !part_lse || !out || !lse) return KDT_ERR_INVALID_ARG;
  if (B <= 0 || q_len <= 0 || H <= 0 || R <= 0 || max_splits <= 0 || split_keys < 0)
    return KDT_ERR_INVALID_ARG;
  if (split_keys > 0 && !prefix_lens) return KDT_ERR_INVALID_ARG;
  if (dtype != KDT_F32 && dtype != KDT_BF16) return KDT_ERR_UNSUPPORTED;
  if (part_dtype != KDT_F32 && part_dtype != KDT_BF16) return KDT_ERR_UNSUPPORTED;
  if (R % (part_dtype == KDT_BF16 ? 16 : 8)) return KDT_ERR_UNSUPPORTED;
  const int64_t vec = dtype == KDT_F32 ? 4 : 8;    // output elements per 16 bytes
  if (!kdt::aligned16(part_o) || !kdt::aligned16(out) || (R % vec) || out_sb % vec || out_st % vec ||
      out_sh % vec || out_sb < 0 || out_st < 0 || out_sh < 0)
    return KDT_ERR_UNSUPPORTED;
  return kdt::launch_merge(dtype, B, q_len, H, R, part_dtype, part_o, part_lse, max_splits, prefix_lens, split_keys, 0, false,
                           out, out_sb, out_st, out_sh, lse, static_cast<hipStream_t>(stream));
}
