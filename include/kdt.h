/*
 * kdt.h — C ABI of libkdt.so: tree-verify MLA-absorb attention for AMD MI355X (gfx950).
 *
 * Pages cited (titles; sections in quotes):
 *   [Checkpoint]  "The Checkpoint: Committing a Working Native DDTree Engine"
 *   [Milestone]   "The Milestone Commit: Cementing a Native DDTree Inference Engine"
 *   [Final]       "The Final Commit: Cementing a Native DDTree Inference Engine for Kimi K2.6"
 *
 * One DDTree verify step, as the pages describe it [Checkpoint, "The Message",
 * KV-cache scheme]: the q_len = 1 + drafts tree tokens [verified_id, drafts]
 * are processed at positions L + depth, the prefix is the cache length L, and
 * the attention mask is [ones over the prefix | tree visibility]; ordinary AR
 * decoding is the q_len = 1 case; after acceptance the accepted path's latents
 * are gathered into place.  Attention runs in the absorbed MLA form [Final,
 * "Input Knowledge Required"]: queries arrive already multiplied by w_kc
 * (q_lat, kv_lora_rank R wide) plus their rope part q_pe (P wide); keys are the
 * cached latents c_kv (R) and rope keys k_pe (P); the result is the latent
 * context, to which w_vc is applied downstream.
 *
 * General rules for every entry point
 *   - Pointers are DEVICE pointers unless stated otherwise.  `stream` is a
 *     hipStream_t passed as void* (NULL = the default stream).  Every call only
 *     enqueues work on `stream`: nothing is synchronised, nothing is allocated or
 *     freed, and no pointer is kept after the call returns.  The library is
 *     stateless; calls from several host threads are safe.
 *   - The caller owns every buffer, including the verify workspace.
 *   - Host-checkable faults (null pointers, non-positive sizes, unsupported
 *     shapes or dtypes, misaligned buffers, a too-small workspace, capacity
 *     below max_prefix_len + q_len) return a nonzero kdt_status and launch
 *     nothing.  A failed kernel launch returns KDT_ERR_LAUNCH.
 *   - Data-dependent faults visible only on the device never cause an access
 *     out of bounds: the kernels clamp, skip the affected work, and OR a
 *     KDT_SEQ_* flag into seq_status[b] when a seq_status array is given
 *     (entry points never clear seq_status; the caller zeroes it).
 */
#ifndef KDT_H
#define KDT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDT_ABI_VERSION 5
#define KDT_MAX_Q_LEN 128           /* tree tokens per sequence (two 64-bit mask words) */

typedef enum {
  KDT_OK = 0,
  KDT_ERR_INVALID_ARG = 1,   /* null pointer, bad size, aliasing that is not allowed */
  KDT_ERR_UNSUPPORTED = 2,   /* dtype / (R, P) / q_len / alignment this build does not handle */
  KDT_ERR_WORKSPACE = 3,     /* workspace missing or smaller than kdt_verify_get_plan reports */
  KDT_ERR_LAUNCH = 4         /* the HIP runtime rejected a kernel launch */
} kdt_status;

typedef enum { KDT_F32 = 0, KDT_BF16 = 1 } kdt_dtype;

/* Per-sequence device status flags (OR-ed into seq_status[b]). */
enum {
  KDT_SEQ_OK = 0,
  KDT_SEQ_BAD_TREE = 1,   /* parent[0] != -1 or parent[i] not in [0, i) */
  KDT_SEQ_BAD_LEN = 2,    /* prefix_len < 0, > max_prefix_len, or prefix_len + q_len > capacity */
  KDT_SEQ_BAD_INDEX = 4   /* an accepted index outside [0, q_len) or n_accepted outside [0, max_acc] */
};

int kdt_abi_version(void);
const char* kdt_status_str(int code);            /* static string, never NULL */

/* ------------------------------------------------------------------------
 * kdt_build_visibility — ancestor-or-self bitmask of every tree node.
 * [Milestone, "The Reasoning Behind the Architecture"]: a node's mask is its
 * parent's mask plus its own bit; two 64-bit words cover up to 65 nodes.
 *
 *   parents  int32 [B, q_len], row-major.  parent[b][0] = -1 (the verified
 *            token); 0 <= parent[b][i] < i otherwise (best-first node order).
 *   vis      uint64 [B, q_len, W] out, W = (q_len + 63) / 64.  Bit (j % 64) of
 *            word j / 64 in row i is set iff node j is node i or an ancestor of
 *            it.  Bits at or above q_len are zero.  Every word is written.
 *   depth    int32 [B, q_len] out, nullable: number of ancestors of node i.
 *   seq_status int32 [B], nullable.
 * A node whose parent is invalid is treated as a root (its row then holds
 * itself and its valid ancestors only) and KDT_SEQ_BAD_TREE is flagged.
 * Supported: 1 <= q_len <= KDT_MAX_Q_LEN, B >= 1.
 * ---------------------------------------------------------------------- */
int kdt_build_visibility(const int32_t* parents, int32_t B, int32_t q_len,
                         uint64_t* vis, int32_t* depth, int32_t* seq_status, void* stream);

/* ------------------------------------------------------------------------
 * kdt_verify_attn — tree-verify attention in latent space.
 * [Checkpoint, "The Message"] KV-cache scheme; [Final, "Input Knowledge
 * Required"] absorbed MLA form.
 *
 * For sequence b with prefix length L = prefix_lens[b], tree token t and head
 * h, the visible keys are cache rows 0..L-1 (the prefix) and rows L+j for every
 * node j with bit j set in vis[b][t] (tree node j's latents sit in row L+j).
 * With s_j = softmax_scale * (q_lat[b,t,h,:] . c_kv[b,j,:] + q_pe[b,t,h,:] . k_pe[b,j,:]):
 *     out[b,t,h,:] = sum_j softmax(s)_j * c_kv[b,j,:]
 *     lse[b,t,h]   = ln sum_j exp(s_j)                (natural log, scale included)
 * q_len = 1 with vis = {1} is one AR decode step.
 *
 * Layouts (strides are in ELEMENTS; the innermost dimension is contiguous):
 *   q_lat [B, q_len, H, R]   strides q_lat_sb, q_lat_st, q_lat_sh
 *   q_pe  [B, q_len, H, P]   strides q_pe_sb,  q_pe_st,  q_pe_sh
 *   c_kv  [B, capacity, R]   strides c_kv_sb, c_kv_ss (row stride may be R+P for a fused [c_kv | k_pe] cache)
 *   k_pe  [B, capacity, P]   strides k_pe_sb, k_pe_ss
 *   vis   uint64 [B, q_len, W] contiguous (as written by kdt_build_visibility),
 *         or NULL: then `parents` (int32 [B, q_len] contiguous, as for
 *         kdt_build_visibility) is required and the split kernel derives the
 *         same masks itself, with the same treatment of invalid parents
 *         (flagged KDT_SEQ_BAD_TREE in seq_status; a sequence skipped for its
 *         prefix length is not examined); this saves the separate visibility
 *         launch.  When vis is given, parents is ignored.
 *   out   [B, q_len, H, R]   in `dtype`, strides out_sb, out_st, out_sh
 *   lse   float32 [B, q_len, H] contiguous
 * `dtype` is the element type of q_lat, q_pe, c_kv, k_pe and out.  Arithmetic:
 * products accumulate in fp32 on the matrix cores; for bf16 the softmax
 * weights are rounded to bf16 before the value contraction; out is rounded to
 * `dtype` (round to nearest even) from fp32.
 * Supported: (dtype, R, P) in {(bf16, 512, 64), (bf16, 64, 16), (f32, 64, 16)};
 * 1 <= q_len <= KDT_MAX_Q_LEN; H >= 1; B >= 1; every input pointer and every
 * row stride 16-byte aligned; capacity >= max_prefix_len + q_len.
 * `max_prefix_len` is a HOST upper bound on prefix_lens[] (it sizes the grid);
 * a sequence with prefix_lens[b] > max_prefix_len, < 0, or prefix_lens[b] +
 * q_len > capacity is skipped (out rows zero, lse = -inf) and flagged
 * KDT_SEQ_BAD_LEN.
 *
 * Split-prefix execution.  The key range of each sequence is cut into splits.
 * With `split_keys` a multiple of 32 (the key tile) every split has split_keys
 * keys.  With 0 (the library's choice) the splits are adaptive: the plan
 * chooses max_splits splits for the longest sequence the launch allows
 * (tiles_max = ceil((max_prefix_len + q_len) / 32) key tiles), and a sequence of
 * T = ceil((prefix_lens[b] + q_len) / 32) tiles gets w = ceil(T * max_splits /
 * tiles_max) splits' worth of tiles, tps = ceil(T / w) tiles per split, split s
 * covering tiles [s * tps, min(T, (s + 1) * tps)) (ceil(T / tps) splits), so
 * that short and long sequences alike give every split workgroup about the
 * same work; total_prefix_len lets the plan count the workgroups that really
 * have work.  split_keys cache rows of either region (c_kv_ss or k_pe_ss
 * elements apart) must span less than 2^31 bytes, or the call returns
 * KDT_ERR_UNSUPPORTED; the library's choice stays within that.
 * Each split produces a normalised partial output and its log-sum-exp in the
 * workspace, and the splits are merged by the log-sum-exp identity.  When every
 * sequence fits in one split there is no merge: the kernel writes out/lse
 * directly.  Otherwise a second kernel does the merge (merge_mode 0, the
 * default), or, with merge_mode 1 and a launch whose workgroups all fit on the
 * device's compute units at once (one per unit), the merge runs inside the
 * same kernel: the split workgroups of a row tile meet at a state word in the
 * workspace, wait for one another for at most merge_wait_us microseconds, and
 * share the merge; a workgroup that stops waiting leaves its share to the last
 * one to arrive, so every call completes whatever the scheduling.  The result
 * is the same bit for bit either way.  (One launch instead of two, but on
 * MI355X the hand-offs between compute units of different XCDs cost more than
 * the second launch saves, so it is not the default.)
 *
 * Workgroup layout (`layout`): 1 = a workgroup owns 128 rows (q_len*H rows of
 * one sequence), each of its four waves 32 rows and all R output columns;
 * 2 = a workgroup owns 64 rows, each pair of waves shares 32 rows and splits
 * the output columns (half the value work per wave, the score work done by
 * both); 3 = as 2, but the two waves of a pair each contract half of the score
 * depth (R + P) and add each other's partial scores through LDS (no score work
 * repeated, one more workgroup barrier per key tile); 4 = a workgroup owns 64
 * rows as two row blocks x two key streams: each wave owns all R output
 * columns of its 32 rows and takes every other key tile, and the two streams
 * of a row block are combined after the last tile.  Layouts 3 and 4: bf16
 * with R = 512 and P = 64 only, KDT_ERR_UNSUPPORTED otherwise.  0 lets the
 * library choose among 1, 2 and 4 (and the split size) by modelling the
 * launch; results agree between layouts to rounding.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t dtype;                       /* kdt_dtype */
  int32_t B, q_len, H, R, P;
  const void* q_lat; int64_t q_lat_sb, q_lat_st, q_lat_sh;
  const void* q_pe;  int64_t q_pe_sb,  q_pe_st,  q_pe_sh;
  const void* c_kv;  int64_t c_kv_sb,  c_kv_ss;
  const void* k_pe;  int64_t k_pe_sb,  k_pe_ss;
  int64_t capacity;                    /* cache rows per sequence */
  const int32_t* prefix_lens;          /* device int32 [B] */
  int32_t max_prefix_len;              /* host upper bound on prefix_lens[] */
  const uint64_t* vis;                 /* device uint64 [B, q_len, W] */
  float softmax_scale;
  void* out; int64_t out_sb, out_st, out_sh;
  float* lse;                          /* device float32 [B, q_len, H] */
  int32_t* seq_status;                 /* device int32 [B], nullable */
  int32_t split_keys;                  /* 0 = auto, else a multiple of 32 */
  int32_t layout;                      /* 0 = auto, 1 = 128-row, 2 = 64-row column split, 3 = 64-row depth split, 4 = 64-row key streams */
  int32_t partials_f32;                /* 1 = keep split partial outputs in float32; 0 = in the input dtype */
  const int32_t* parents;              /* device int32 [B, q_len]; used when vis is NULL */
  int32_t merge_mode;                  /* 0 = separate merge kernel, 1 = merge inside the split kernel when the launch allows */
  int32_t merge_wait_us;               /* longest wait of a split workgroup for the rest of its row tile
                                          (0 = the default, 2000; < 0 = no wait, the last one out merges
                                          whatever was left: for tests of that path) */
  int64_t total_prefix_len;            /* host hint, sum of prefix_lens[] (0 = unknown: taken as
                                          B * max_prefix_len); only the plan depends on it */
  int32_t schedule;                    /* 0 = the library's choice, 1 = splits (fixed or adaptive),
                                          2 = the balanced schedule (below; split_keys must be 0) */
  int32_t gang_size;                   /* balanced schedule: row tiles per gang (0 = the library's choice) */
} kdt_verify_desc;

/* Host-only planning: no device memory is touched (the compute-unit count of
 * the current device is queried once per device).  The partial buffers live
 * in the workspace at the given byte offsets:
 *   part_o   part_dtype [B, max_splits, NBLK, 32*R]  normalised partial outputs, tiled
 *   part_lse float32 [B, max_splits, q_len*H]        natural-log partial LSE (-inf: empty split)
 * Row index within a sequence is m = t*H + h.  NBLK = ceil(q_len*H / 32): rows
 * are grouped in blocks of 32, and inside block m / 32 element (m, c) sits at
 *   float32:  256*(c/8) + 128*((c/4)%2) + 4*(m%32) + c%4
 *   bf16:     512*(c/16) + 8*(m%32 + 32*((c/4)%2)) + 4*((c/8)%2) + c%4
 * (elements), the register order of a 32x32 matrix-core accumulator, so the
 * split kernel writes whole cache lines (each lane 16 bytes, each store
 * instruction one contiguous 1 KB run).  Padding rows of the last block hold
 * unspecified values.  part_dtype is KDT_F32 for float32 inputs or when
 * partials_f32 is set, else KDT_BF16 (rounded to nearest even: one more
 * rounding of the output's own precision, which halves the partial traffic).
 * Sequence b uses splits 0 .. n_b - 1, n_b = ceil((prefix_lens[b] + q_len) /
 * split_keys) for fixed splits (tiles_max == 0), the adaptive count above, or
 * the count the balanced schedule gives each of its row-tile groups (below);
 * the part_lse rows of its other splits are written -inf by kdt_verify_partials
 * (so a merge over all max_splits splits is always right).
 * Balanced schedule (gang_size > 0; stream-K style): the row tiles of a
 * sequence form groups of gang_size consecutive tiles, and every (sequence,
 * group) pair is a stream of piece_units units (the start-up of its first
 * piece) followed by T_b = ceil((prefix_lens[b] + q_len) / 32) key-tile units
 * (a sequence with an invalid prefix length: one unit).  The streams, laid end
 * to end in sequence order, U units in all, are cut into ranges of A =
 * max(ceil(U / gangs), ceil(T_max / (max_splits - 1))) units (T_max the most
 * key tiles of a valid sequence; A is at most the key tiles one piece may
 * span); range j goes to gang j mod gangs, a gang being gang_size workgroups
 * that each take one row tile of the group and move through the same keys
 * together.  The grid is gangs * gang_size workgroups, one per compute unit,
 * so the work is even however the lengths are mixed.  The key tiles of a
 * stream inside range j are partial j - floor(r / A) of the stream's rows, r
 * its first key-tile unit; a range holding only start-up units of a stream
 * holds no piece of it.  Merge such partials with split_keys == 0.  The walk
 * counts units in 32 bits: a batch whose units could exceed 2e9 (B times the
 * longest stream) is not given the balanced schedule (KDT_ERR_UNSUPPORTED when
 * it is asked for).
 * Merge state (when the merge is fused): one 32-bit word per row tile, uint32
 * [B, NRT] at counter_offset, NRT = ceil(q_len*H / rows per workgroup of the
 * layout): two counts and a generation bit.  The words must be zero before
 * the first kdt_verify_attn call that uses the workspace (allocate it zeroed);
 * every call leaves the counts at zero again (the generation bit alternates),
 * so one workspace serves any sequence of calls on one stream.  Calls that
 * share a workspace must not overlap in time. */
typedef struct {
  int32_t split_keys;          /* keys per split (multiple of 32); balanced schedule: about the keys of
                                  one range, as planned from total_prefix_len (for information) */
  int32_t max_splits;          /* ceil((max_prefix_len + q_len) / split_keys) */
  int32_t rows;                /* q_len * H */
  int32_t direct;              /* 1: max_splits == 1, no partials, no merge */
  int32_t layout;              /* workgroup layout used: 1 to 4 */
  int32_t part_dtype;          /* kdt_dtype of part_o */
  int64_t part_o_offset;       /* bytes into the workspace */
  int64_t part_lse_offset;
  size_t workspace_bytes;      /* what kdt_verify_attn needs: 0 when direct, else partials and counters */
  size_t partials_bytes;       /* what kdt_verify_partials needs (part_o and part_lse; also when direct) */
  int32_t fused_merge;         /* 1: kdt_verify_attn merges inside the split kernel (one launch) */
  int32_t tiles_max;           /* > 0: adaptive splits (above), the longest sequence's key tiles; 0: fixed */
  int64_t counter_offset;      /* bytes into the workspace of the merge counters */
  int32_t gang_size;           /* > 0: the balanced schedule (above), row tiles per gang; 0: splits */
  int32_t gangs;               /* balanced schedule: gangs in the launch */
  int32_t piece_units;         /* balanced schedule: start-up units charged to every stream (below) */
  int32_t reserved;
} kdt_verify_plan;

int kdt_verify_get_plan(const kdt_verify_desc* d, kdt_verify_plan* plan);

/* Full verify: split stage and merge (or direct output when one split
 * suffices).  `workspace` may be NULL only when the plan says workspace_bytes
 * == 0; its merge counters must be zero before its first use (see above). */
int kdt_verify_attn(const kdt_verify_desc* d, void* workspace, size_t ws_bytes, void* stream);

/* Split stage only: always writes the partial buffers (part_o, part_lse) in the
 * workspace (at least plan.partials_bytes), even when one split would do;
 * `out`/`lse` are not touched and nothing is merged. */
int kdt_verify_partials(const kdt_verify_desc* d, void* workspace, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation as kdt_verify_attn, with the workspace taken from a fixed
 * device array inside the library instead of from the caller.  Each GPU that
 * loads the library holds its own copy of that array (KDT_NOALLOC_MAX_WORKSPACE
 * bytes) until the process ends; its address is looked up once per device, on
 * the first call with that device current.  Nothing is allocated or freed.
 * Every call on one GPU uses the same array, so calls that overlap in time on
 * one GPU (several streams, several host threads) race and must be
 * serialised by the caller.  Returns KDT_ERR_WORKSPACE when the plan's
 * workspace_bytes exceeds KDT_NOALLOC_MAX_WORKSPACE (force a larger
 * split_keys, or use kdt_verify_attn), and KDT_ERR_UNSUPPORTED for
 * merge_mode 1 (its state words would have to start at zero). */
#define KDT_NOALLOC_MAX_WORKSPACE ((size_t)32 << 20)
int kdt_verify_attn_noalloc(const kdt_verify_desc* d, void* stream);

/* ------------------------------------------------------------------------
 * kdt_merge_partials — cross-split log-sum-exp merge.
 *   lse[b,m] = ln sum_k exp(part_lse[b,k,m]);
 *   out[b,m,:] = sum_k exp(part_lse[b,k,m] - lse[b,m]) * part_o[b,k,m,:]
 * over k < n_splits, where n_splits = max_splits when split_keys == 0, else
 * ceil((prefix_lens[b] + q_len) / split_keys) clamped to [1, max_splits]
 * (partials of adaptive splits or of the balanced schedule: merge with
 * split_keys == 0).
 * Splits with part_lse = -inf carry no weight; a row with no finite split gets
 * out = 0 and lse = -inf.  out is written in `dtype` (bf16: round to nearest
 * even).  part_o (elements of `part_dtype`, KDT_F32 or KDT_BF16) and part_lse
 * are contiguous with the layout given above (tiled part_o); out has strides
 * out_sb, out_st, out_sh (elements) over [B, q_len, H, R].  R must be a
 * multiple of 8 (of 16 for bf16 partials).
 * prefix_lens may be NULL when split_keys == 0.
 * ---------------------------------------------------------------------- */
int kdt_merge_partials(int32_t dtype, int32_t B, int32_t q_len, int32_t H, int32_t R, int32_t part_dtype,
                       const void* part_o, const float* part_lse, int32_t max_splits,
                       const int32_t* prefix_lens, int32_t split_keys,
                       void* out, int64_t out_sb, int64_t out_st, int64_t out_sh,
                       float* lse, void* stream);

/* ------------------------------------------------------------------------
 * kdt_gather_accepted — post-accept compaction of the accepted path's latents.
 * [Checkpoint, "The Message"]: once the tree is accepted, the latents of the
 * accepted path are gathered into the rows right after the prefix (the KV
 * cache scheme's compaction after the verify).
 *
 * For every layer l < num_layers, sequence b and k < n_accepted[b]:
 *     row L_b + k  <-  (previous contents of) row L_b + accepted[b, k]
 * where L_b = prefix_lens[b].  All rows are read before any is written, so
 * overlapping source and destination rows are safe; no other row changes.
 *   cache      base of layer 0; element (l, b, s, c) at
 *              l*layer_stride + b*cache_sb + s*cache_ss + c   (elements of `dtype`)
 *   row_elems  elements copied per row (e.g. R + P for a fused cache row)
 *   accepted   int32 [B, max_acc] row-major; n_accepted int32 [B]
 *   new_prefix_lens  int32 [B] out, nullable: L_b + n_accepted[b].  Must not
 *              alias prefix_lens.
 * Device checks: a sequence with L_b < 0 or L_b + q_len > capacity is skipped
 * (KDT_SEQ_BAD_LEN); n_accepted outside [0, min(max_acc, q_len)] is clamped
 * and an accepted index outside [0, q_len) skips that row (KDT_SEQ_BAD_INDEX).
 * The copy is bit-exact.  Supported: 1 <= q_len <= KDT_MAX_Q_LEN, 1 <= max_acc <= q_len.
 * ---------------------------------------------------------------------- */
int kdt_gather_accepted(int32_t dtype, int32_t B, int32_t q_len, int32_t row_elems,
                        void* cache, int64_t cache_sb, int64_t cache_ss, int64_t capacity,
                        int32_t num_layers, int64_t layer_stride,
                        const int32_t* prefix_lens, const int32_t* accepted,
                        const int32_t* n_accepted, int32_t max_acc,
                        int32_t* new_prefix_lens, int32_t* seq_status, void* stream);

/* ------------------------------------------------------------------------
 * kdt_tree_accept — greedy acceptance of a verified draft tree.
 * [Checkpoint, "The Message"]: the decode loop runs tree build -> verify ->
 * tree accept -> cache compaction, and greedy tree decoding reproduces greedy
 * autoregressive decoding token for token; [Milestone, "Mistakes and
 * Incorrect Assumptions"]: walks are bounded (cyclic inputs cannot hang).
 *
 * For each sequence b, starting at node 0 (the verified token), repeatedly
 * move to the lowest-index child c of the current node u with
 * tokens[b][c] == target_pred[b][u]; stop when no child matches.
 *   parents      int32 [B, q_len]  (as for kdt_build_visibility)
 *   tokens       int32 [B, q_len]  draft token of each node (node 0: the verified token)
 *   target_pred  int32 [B, q_len]  the target model's greedy next token after each node
 *   accepted     int32 [B, q_len]  out: visited nodes from the root, -1 after the last;
 *                                  pass it with max_acc = q_len to kdt_gather_accepted
 *   n_accepted   int32 [B]         out: path length (>= 1, the root is always accepted)
 *   bonus        int32 [B]         out, nullable: target_pred at the last accepted node
 *   seq_status   int32 [B]         nullable; a node whose parent is not an earlier
 *                                  node (or node 0 with a parent) is unreachable and
 *                                  KDT_SEQ_BAD_TREE is flagged
 * Supported: 1 <= q_len <= KDT_MAX_Q_LEN, B >= 1.  The result is exact
 * (integer comparisons only).
 * ---------------------------------------------------------------------- */
int kdt_tree_accept(const int32_t* parents, const int32_t* tokens, const int32_t* target_pred,
                    int32_t B, int32_t q_len, int32_t* accepted, int32_t* n_accepted,
                    int32_t* bonus, int32_t* seq_status, void* stream);

/* ------------------------------------------------------------------------
 * kdt_build_tree — best-first draft tree from the drafter's top-k lists.
 * [Milestone, "The Context: Why This Commit Exists"]: the tree was built on
 * the host with a heap (a device-host round trip per decode step); here it is
 * built on the device.  [Milestone, "The Reasoning Behind the Architecture"]:
 * one work unit per request, double-precision logw, first-child /
 * next-sibling links sorted by log-probability.  [Final, "Input Knowledge
 * Required"]: best-first from top-k logits.
 *
 * For draft position d = 1..D the drafter gives its K best tokens with
 * log-probabilities, best first; every node at depth d - 1 has those K tokens
 * as candidate children.  The root (node 0) is the verified token with logw
 * 0; a child of rank j has logw = logw(parent) + logprob[d][j] (double).
 * Nodes are created as by a plain heap onto which every created node pushes
 * all K of its children: in order of decreasing logw until q_len nodes exist
 * or no candidate remains, equal logw going to the child of the earlier
 * created parent, then to the lower rank (the push order).  The device holds
 * only each parent's best remaining child, which gives the same tree because
 * the log-probabilities are sorted best first (the result is unspecified for
 * unsorted lists).  Budget slots left over are padding: parent 0, token -1,
 * depth 1, logw -inf, no links.
 *   topk_tokens    int32 [B, D, K]   (read only)
 *   topk_logprobs  float [B, D, K]   sorted best first per position (read only)
 *   root_tokens    int32 [B]         the verified token of each request
 *   parents        int32 [B, q_len]  out: -1 for the root, else an earlier node
 *                                    (valid input for kdt_build_visibility)
 *   tokens         int32 [B, q_len]  out: draft token of each node (root: root_tokens)
 *   depth          int32 [B, q_len]  out
 *   logw           double [B, q_len] out, nullable
 *   first_child, next_sibling  int32 [B, q_len]  out, nullable (-1: none)
 *   n_nodes        int32 [B]         out, nullable: created nodes (<= q_len)
 * Supported: 1 <= q_len <= KDT_MAX_Q_LEN; D, K >= 1; K <= 64 unless q_len <= 64.
 * The result is exact (the same double additions and comparisons in the same
 * order as the definition).
 * ---------------------------------------------------------------------- */
int kdt_build_tree(const int32_t* topk_tokens, const float* topk_logprobs, const int32_t* root_tokens,
                   int32_t B, int32_t D, int32_t K, int32_t q_len, int32_t* parents, int32_t* tokens,
                   int32_t* depth, double* logw, int32_t* first_child, int32_t* next_sibling,
                   int32_t* n_nodes, void* stream);

/* ------------------------------------------------------------------------
 * The steps on either side of the verify [Checkpoint, "The Message": split_q,
 * absorb_qk / absorb_vc, rope, cache append, positions L + depth; Final,
 * "Input Knowledge Required": absorb form].  bf16 in and out, fp32 (rotary
 * angles: fp64) inside.  Positions: node t of sequence b sits at
 * prefix_lens[b] + depth[b, t] (depth int32 [B, T], e.g. from
 * kdt_build_visibility or kdt_build_tree).  NeoX rotary embedding: for
 * i < P/2 the pair (x[i], x[i + P/2]) turns by pos * rope_theta^(-2i/P).
 *
 * kdt_absorb_q: q [B, T, H, dn + P] (element strides q_sb, q_st, q_sh, each a
 *   multiple of 8; innermost contiguous) is split per head into its first dn
 *   values and its last P values;
 *     q_lat[b, t, h, r] = sum_i w_kc_t[h, r, i] * q[b, t, h, i]   (i < dn)
 *     q_pe[b, t, h, :]  = rope(q[b, t, h, dn:], pos(b, t))
 *   w_kc_t [H, R, dn] contiguous (the key up-projection of each head,
 *   transposed); q_lat [B, T, H, R] and q_pe [B, T, H, P] contiguous outputs
 *   (the verify's query inputs).  Supported: dtype KDT_BF16, dn in {32, 64,
 *   128, 256, 512}, R a multiple of 32 * (4, 4, 4, 2, 1) respectively, P even,
 *   16-byte aligned q, w_kc_t, q_lat.
 * kdt_absorb_o: o[b, t, h, j] = sum_r w_vc[h, j, r] * o_lat[b, t, h, r];
 *   o_lat [B, T, H, R], w_vc [H, dv, R], o [B, T, H, dv], all contiguous and
 *   16-byte aligned.  Supported: R in {32, 64, 128, 256, 512}, dv a multiple
 *   of 32 * (4, 4, 4, 2, 1) respectively.
 * kdt_append_tree_kv: cache row prefix_lens[b] + t of sequence b (cache
 *   [B, capacity, >= R + P], element strides cache_sb, cache_ss) gets
 *   [c_kv_new[b, t] (R) | rope(k_rope_new[b, t], pos(b, t)) (P)];
 *   c_kv_new [B, T, R], k_rope_new [B, T, P] contiguous.  A sequence with
 *   prefix_lens[b] + T > capacity (or < 0) is skipped and flagged
 *   KDT_SEQ_BAD_LEN in seq_status (nullable).
 * All three are asynchronous on `stream` and keep no pointer.
 * ---------------------------------------------------------------------- */
int kdt_absorb_q(int32_t dtype, int32_t B, int32_t T, int32_t H, int32_t dn, int32_t P, int32_t R,
                 const void* q, int64_t q_sb, int64_t q_st, int64_t q_sh, const void* w_kc_t,
                 const int32_t* prefix_lens, const int32_t* depth, float rope_theta, void* q_lat,
                 void* q_pe, void* stream);
int kdt_absorb_o(int32_t dtype, int32_t B, int32_t T, int32_t H, int32_t R, int32_t dv,
                 const void* o_lat, const void* w_vc, void* o, void* stream);
int kdt_append_tree_kv(int32_t dtype, int32_t B, int32_t T, int32_t R, int32_t P, const void* c_kv_new,
                       const void* k_rope_new, const int32_t* prefix_lens, const int32_t* depth,
                       float rope_theta, void* cache, int64_t cache_sb, int64_t cache_ss,
                       int64_t capacity, int32_t* seq_status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDT_H */
