// The steps on either side of the verify attention: the query split with the
// key absorb and rotary embedding, the cache append of the tree tokens, and
// the value absorb.
//
// "The Checkpoint: Committing a Working Native DDTree Engine", section "The
// Message": the engine's ops include split_q, absorb_qk / absorb_vc and rope,
// the tree tokens are processed at positions L + depth, and the cache is
// appended before the verify; "The Final Commit: Cementing a Native DDTree
// Inference Engine for Kimi K2.6", section "Input Knowledge Required": the
// absorb form of MLA (w_kc, w_vc).
//
//  * absorb_q:  q_lat[m, h, :] = w_kc_t[h] (R x dn) . q[m, h, :dn], and
//               q_pe[m, h, :] = NeoX rope of q[m, h, dn:] at L_b + depth(t),
//    for rows m = (b, t), in one launch (the rope in the same workgroups).
//  * absorb_o:  o[m, h, :] = w_vc[h] (dv x R) . o_lat[m, h, :].
//  * append:    cache row L_b + t gets the token's latent and its rotary key
//               rotated at L_b + depth(t).
//
// Both absorbs are one contraction per head with the weight row contiguous
// along the contraction; they run on v_mfma_f32_32x32x16_bf16 as the
// transposed product C^T = W . X^T, so that a lane ends up holding four
// consecutive outputs of one row (8-byte stores).  A workgroup owns one head
// and NCB 32-wide blocks of outputs for a group of up to kAbsorbRowBlocks
// 32-row blocks, and keeps its weight operands for the whole contraction in
// registers; its four waves take the row blocks in turn.
#include <math.h>

#include "kdt_common.hpp"

namespace kdt {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kAbsorbRowBlocks = 8;             // 32-row blocks per workgroup (two per wave)

// Row source of a contraction: element (row m, k) of head h.
struct RowSrc {
  const __bf16* base;
  int64_t sb, st, sh;   // element strides of batch, token, head
  int T;
  __device__ __forceinline__ const __bf16* row(int m, int h) const {
    const int b = m / T, t = m - b * T;
    return base + b * sb + t * st + h * sh;
  }
};

// Rotation of pair i at position pos: the pair (x[i], x[i + P/2]) turns by
// pos * theta^(-2i/P).  The angle is formed and reduced to [-pi, pi] in double
// precision (positions reach 10^5 and more); the sine and cosine of the
// reduced angle are taken in single precision.
__device__ __forceinline__ void rope_angle(int P, int i, double pos, double log2_theta, float& c, float& s) {
  const double ang = pos * exp2(-(2.0 * i / P) * log2_theta);
  const double two_pi = 6.283185307179586476925286766559;
  const float red = (float)(ang - two_pi * rint(ang / two_pi));
  s = sinf(red);
  c = cosf(red);
}

__device__ __forceinline__ void rope_apply(const __bf16* src, __bf16* dst, int half, int i, float c, float s) {
  const float x1 = (float)src[i], x2 = (float)src[i + half];
  dst[i] = (__bf16)(x1 * c - x2 * s);
  dst[i + half] = (__bf16)(x2 * c + x1 * s);
}

// The rotary part of the query split, done by the absorb_q launch itself:
// q_pe[b, t, h, :] = rope(q[b, t, h, dn:], L_b + depth[b, t]) (off when q_pe
// is null, as for absorb_o).
struct RopeArgs {
  const int32_t* prefix_lens;
  const int32_t* depth;
  double log2_theta;
  __bf16* q_pe;
  int dn, P;
};

// C^T[n][m] = sum_k W[h][n][k] X[m][k]; W is [H, N, K] contiguous, the output
// [rows, H, N] contiguous.  KS = K / 16 contraction steps, NCB output blocks
// of 32 per workgroup (their weight fragments stay in registers).  With
// rope.q_pe set, the workgroups of head h and row group z also rotate the
// query's rope part for those rows, the pairs shared among the gridDim.y
// workgroups of the group.
template <int KS, int NCB>
__global__ __launch_bounds__(256) void absorb_gemm_kernel(RowSrc x, const __bf16* __restrict__ w, int M, int H,
                                                          int N, __bf16* __restrict__ out, RopeArgs rope) {
  constexpr int K = KS * 16;
  const int h = blockIdx.x;
  const int nb0 = blockIdx.y * NCB;            // first 32-wide output block of this workgroup
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 31, hh = lane >> 5;

  // weight operands: A[n][k] for n = 32 (nb0 + cb) + r, k = 16 c + 8 hh .. + 7
  bf16x8_t wf[NCB][KS];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const __bf16* wr = w + ((int64_t)h * N + 32 * (nb0 + cb) + r) * K + 8 * hh;
#pragma unroll
    for (int c = 0; c < KS; ++c) wf[cb][c] = *reinterpret_cast<const bf16x8_t*>(wr + 16 * c);
  }
  const int n_rb = min((M + 31) / 32, (int)(blockIdx.z + 1) * kAbsorbRowBlocks);
#pragma unroll 1
  for (int rb = blockIdx.z * kAbsorbRowBlocks + wave; rb < n_rb; rb += 4) {
    const int m = rb * 32 + r;
    const bool ok = m < M;
    const __bf16* xr = x.row(ok ? m : 0, h) + 8 * hh;
    f32x16_t acc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[cb][v] = 0.0f;
#pragma unroll
    for (int c = 0; c < KS; ++c) {
      const bf16x8_t xf = *reinterpret_cast<const bf16x8_t*>(xr + 16 * c);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cb][c], xf, acc[cb], 0, 0, 0);
    }
    if (!ok) continue;
    // lane (r, hh) holds outputs n = 32 (nb0 + cb) + 8 g + 4 hh + e of row m
    __bf16* o = out + ((int64_t)m * H + h) * N + 32 * nb0 + 4 * hh;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<bf16x4_t*>(o + 32 * cb + 8 * g) =
            bf16x4_t{(__bf16)acc[cb][4 * g], (__bf16)acc[cb][4 * g + 1], (__bf16)acc[cb][4 * g + 2],
                     (__bf16)acc[cb][4 * g + 3]};
  }
  if (rope.q_pe) {
    const int half = rope.P / 2, ny = gridDim.y;
    const int i0 = (int)blockIdx.y * half / ny, np = ((int)blockIdx.y + 1) * half / ny - i0;
    const int m0 = (int)blockIdx.z * kAbsorbRowBlocks * 32, m1 = min(M, m0 + kAbsorbRowBlocks * 32);
    for (int e = threadIdx.x; e < (m1 - m0) * np; e += 256) {
      const int m = m0 + e / np, i = i0 + e % np;
      float c, s;
      rope_angle(rope.P, i, (double)rope.prefix_lens[m / x.T] + (double)rope.depth[m], rope.log2_theta, c, s);
      rope_apply(x.row(m, h) + rope.dn, rope.q_pe + ((int64_t)m * H + h) * rope.P, half, i, c, s);
    }
  }
}

// cache row L_b + t <- [c_kv_new[b, t] | rope(k_rope_new[b, t], L_b + depth[b, t])]
__global__ __launch_bounds__(256) void append_kernel(const __bf16* __restrict__ c_new,
                                                     const __bf16* __restrict__ k_new, int T, int R, int P,
                                                     const int32_t* __restrict__ prefix_lens,
                                                     const int32_t* __restrict__ depth, double log2_theta,
                                                     __bf16* __restrict__ cache, int64_t sb, int64_t ss,
                                                     int64_t capacity, int32_t* __restrict__ seq_status) {
  const int m = blockIdx.x;                     // (b, t)
  const int b = m / T, t = m - b * T;
  const int L = prefix_lens[b];
  if (L < 0 || (int64_t)L + T > capacity) {
    if (t == 0 && threadIdx.x == 0) flag_seq(seq_status, b, KDT_SEQ_BAD_LEN);
    return;
  }
  __bf16* row = cache + b * sb + (int64_t)(L + t) * ss;
  const __bf16* cs = c_new + (int64_t)m * R;
  for (int i = threadIdx.x; i < R; i += blockDim.x) row[i] = cs[i];
  const double pos = (double)L + (double)depth[m];
  for (int i = threadIdx.x; i < P / 2; i += blockDim.x) {
    float c, s;
    rope_angle(P, i, pos, log2_theta, c, s);
    rope_apply(k_new + (int64_t)m * P, row + R, P / 2, i, c, s);
  }
}

template <int KS, int NCB>
static int launch_gemm(const RowSrc& x, const __bf16* w, int M, int H, int N, __bf16* out, const RopeArgs& rope,
                       hipStream_t s) {
  if (N % (32 * NCB)) return KDT_ERR_UNSUPPORTED;
  const int groups = ((M + 31) / 32 + kAbsorbRowBlocks - 1) / kAbsorbRowBlocks;
  if (groups > 65535) return KDT_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((absorb_gemm_kernel<KS, NCB>), dim3(H, N / (32 * NCB), groups), dim3(256), 0, s, x, w, M, H,
                     N, out, rope);
  return launch_status();
}

// dispatch on the contraction length: the weight fragments of a workgroup
// (NCB x KS x 4 registers) stay within 64 registers where possible, so that
// two waves fit on a SIMD
static int gemm(const RowSrc& x, const __bf16* w, int K, int M, int H, int N, __bf16* out, const RopeArgs& rope,
                hipStream_t s) {
  switch (K) {
    case 32: return launch_gemm<2, 2>(x, w, M, H, N, out, rope, s);
    case 64: return launch_gemm<4, 2>(x, w, M, H, N, out, rope, s);
    case 128: return launch_gemm<8, 2>(x, w, M, H, N, out, rope, s);
    case 256: return launch_gemm<16, 1>(x, w, M, H, N, out, rope, s);
    case 512: return launch_gemm<32, 1>(x, w, M, H, N, out, rope, s);
    default: return KDT_ERR_UNSUPPORTED;
  }
}

}  // namespace kdt

extern "C" int kdt_absorb_q(int32_t dtype, int32_t B, int32_t T, int32_t H, int32_t dn, int32_t P, int32_t R,
                            const void* q, int64_t q_sb, int64_t q_st, int64_t q_sh, const void* w_kc_t,
                            const int32_t* prefix_lens, const int32_t* depth, float rope_theta, void* q_lat,
                            void* q_pe, void* stream) {
  if (!q || !w_kc_t || !prefix_lens || !depth || !q_lat || !q_pe) return KDT_ERR_INVALID_ARG;
  if (B <= 0 || T <= 0 || H <= 0 || dn <= 0 || P <= 0 || R <= 0 || q_sb < 0 || q_st < 0 || q_sh < 0)
    return KDT_ERR_INVALID_ARG;
  if (!(rope_theta > 1.0f) || !isfinite(rope_theta)) return KDT_ERR_INVALID_ARG;
  if (dtype != KDT_BF16 || (P & 1)) return KDT_ERR_UNSUPPORTED;
  if (!kdt::aligned16(q) || !kdt::aligned16(w_kc_t) || !kdt::aligned16(q_lat) || (q_sb | q_st | q_sh) & 7)
    return KDT_ERR_UNSUPPORTED;
  if ((int64_t)B * T > 0x7FFFFFFF / 64 || (int64_t)B * T * H * P > 0x7FFFFFFF) return KDT_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const kdt::RowSrc x{static_cast<const __bf16*>(q), q_sb, q_st, q_sh, T};
  const int M = B * T;
  const kdt::RopeArgs rope{prefix_lens, depth, log2((double)rope_theta), static_cast<__bf16*>(q_pe), (int)dn,
                           (int)P};
  return kdt::gemm(x, static_cast<const __bf16*>(w_kc_t), dn, M, H, R, static_cast<__bf16*>(q_lat), rope, s);
}

extern "C" int kdt_absorb_o(int32_t dtype, int32_t B, int32_t T, int32_t H, int32_t R, int32_t dv,
                            const void* o_lat, const void* w_vc, void* o, void* stream) {
  if (!o_lat || !w_vc || !o) return KDT_ERR_INVALID_ARG;
  if (B <= 0 || T <= 0 || H <= 0 || R <= 0 || dv <= 0) return KDT_ERR_INVALID_ARG;
  if (dtype != KDT_BF16) return KDT_ERR_UNSUPPORTED;
  if (!kdt::aligned16(o_lat) || !kdt::aligned16(w_vc) || !kdt::aligned16(o)) return KDT_ERR_UNSUPPORTED;
  if ((int64_t)B * T > 0x7FFFFFFF / 64) return KDT_ERR_UNSUPPORTED;
  const kdt::RowSrc x{static_cast<const __bf16*>(o_lat), (int64_t)T * H * R, (int64_t)H * R, R, T};
  return kdt::gemm(x, static_cast<const __bf16*>(w_vc), R, B * T, H, dv, static_cast<__bf16*>(o),
                   kdt::RopeArgs{nullptr, nullptr, 0.0, nullptr, 0, 0}, static_cast<hipStream_t>(stream));
}

extern "C" int kdt_append_tree_kv(int32_t dtype, int32_t B, int32_t T, int32_t R, int32_t P, const void* c_kv_new,
                                  const void* k_rope_new, const int32_t* prefix_lens, const int32_t* depth,
                                  float rope_theta, void* cache, int64_t cache_sb, int64_t cache_ss,
                                  int64_t capacity, int32_t* seq_status, void* stream) {
  if (!c_kv_new || !k_rope_new || !prefix_lens || !depth || !cache) return KDT_ERR_INVALID_ARG;
  if (B <= 0 || T <= 0 || R <= 0 || P <= 0 || cache_sb < 0 || cache_ss < R + P || capacity < T)
    return KDT_ERR_INVALID_ARG;
  if (!(rope_theta > 1.0f) || !isfinite(rope_theta)) return KDT_ERR_INVALID_ARG;
  if (dtype != KDT_BF16 || (P & 1)) return KDT_ERR_UNSUPPORTED;
  if ((int64_t)B * T > 0x7FFFFFFF) return KDT_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(kdt::append_kernel, dim3(B * T), dim3(256), 0, s, static_cast<const __bf16*>(c_kv_new),
                     static_cast<const __bf16*>(k_rope_new), (int)T, (int)R, (int)P, prefix_lens, depth,
                     log2((double)rope_theta), static_cast<__bf16*>(cache), cache_sb, cache_ss, capacity, seq_status);
  return kdt::launch_status();
}
