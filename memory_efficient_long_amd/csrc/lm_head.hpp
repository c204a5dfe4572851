// Blockwise LM head with cross-entropy loss ("Blockwise Parallel Transformer
// for Long Context Large Models", §3.4, handling of the cross-entropy loss:
// the loss is accumulated block by block so the s x V logits never exist at
// once). The logits of a chunk of rows come from the MFMA GEMM (z W); its
// epilogues here reduce them on the fly:
//
//   forward : per row and 32-column block, the pair (max, sum of 2^(x - max))
//             of x = logit * log2(e), plus the logit at the row's target;
//             ce_combine_kernel merges a row's pairs into its log-sum-exp and
//             loss. Nothing of size rows x V is written.
//   backward: the same GEMM again, with dlogit = g (2^(x - lse2) - [n == t])
//             written for the chunk only, then dz = dlogits W^T and
//             dW += z^T dlogits (ordinary GEMMs).
//   fused   : (forward and backward in one call, the cotangents g known
//             before the forward) the forward's GEMM also stores the chunk's
//             fp32 logits; after the combine, ce_dlogit_kernel forms the
//             chunk's dlogits from them with the backward epilogue's
//             arithmetic, so the logits GEMM runs once per chunk.
//
// Statistics are kept in base 2 (x = logit * log2 e); lse2 is the base-2
// log-sum-exp, loss = lse2 ln 2 - logit[t]. A target outside [0, V) marks an
// ignored row (no loss, no gradient).
#pragma once

#include "gemm.hpp"

namespace bpt {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Merge of two (max, sum) pairs of base-2 partial log-sum-exps (an empty
// pair is (-inf, 0)).
__device__ __forceinline__ void lse_merge(float& m, float& l, float m2, float l2) {
  const float mx = fmaxf(m, m2);
  const float s = l * fast_exp2(m - mx) + l2 * fast_exp2(m2 - mx);
  l = mx == -INFINITY ? 0.f : s;
  m = mx;
}

// Lane value of lane ^ K within each 32-lane half (ds_swizzle in bit-mask
// mode: and 0x1f, or 0, xor K; no LDS memory access).
template <int K>
__device__ __forceinline__ float swz_xor(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                               (K << 10) | 0x1f));
}

// One reduce-scatter step over lanes lane ^ K: of the 2H (max, sum) pairs a
// lane holds, it keeps the H whose index bit matches its lane bit, receives
// the partner's copy of those, and merges them.
template <int K, int H>
__device__ __forceinline__ void rs_step(float (&m)[16], float (&l)[16], int lr) {
  const bool hi = (lr & K) != 0;
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const float sm = hi ? m[i] : m[i + H], sl = hi ? l[i] : l[i + H];
    const float km = hi ? m[i + H] : m[i], kl = hi ? l[i + H] : l[i];
    const float rm = swz_xor<K>(sm), rl = swz_xor<K>(sl);
    m[i] = km;
    l[i] = kl;
    lse_merge(m[i], l[i], rm, rl);
  }
}

// Forward epilogue: log-sum-exp partials per (row, 32-column block) and the
// target logit of each row; STORE: the fp32 logits too (the fused call).
template <bool STORE = false>
struct EpiCEStats {
  float2* part;        // [M, nb]: (max, sum) in base-2 units
  int64_t nb;          // 32-column blocks per row
  float* tlogit;       // [M]: logit of the row's target (raw, natural units)
  const int* targets;  // [M]
  int V;               // vocabulary size (columns >= V are not logits)
  float* logits;       // STORE: [M, V] raw logits (row stride V)
  static constexpr bool kPair = false;
  struct Col {};
  struct Pre {};
};

// The 32 x 32 block of a lane's accumulators: this lane holds column `col`
// of rows m0 + acc_row(r, g), r < 16. A reduce-scatter over the 32 lanes of
// the half-wave leaves lanes lr and lr ^ 1 with row (lr >> 1) merged over all
// 32 columns; the even one stores the pair.
template <bool EVEN, bool STORE>
__device__ __forceinline__ void epilogue_block(const EpiCEStats<STORE>& e, const f32x16& acc,
                                               int m0, int col, int g, int M, int) {
  const int lr = col & 31;  // block columns start at multiples of 32
  const bool cvalid = col < e.V;
  int tg[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) tg[r] = e.targets[min(m0 + acc_row(r, g), M - 1)];
  float m[16], l[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    m[r] = cvalid ? acc[r] * kLog2e : -INFINITY;
    l[r] = cvalid ? 1.f : 0.f;
  }
  // The target logits: a row's target falls in one 32-column block of the
  // ~V / 32, so almost every wave skips the per-element stores on one test.
  bool hit = false;
#pragma unroll
  for (int r = 0; r < 16; ++r) hit |= tg[r] == col;
  if (__any(hit) && cvalid) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + acc_row(r, g);
      if (row < M && tg[r] == col) e.tlogit[row] = acc[r];
    }
  }
  if constexpr (STORE) {
    // cvalid and m0 + 32 <= M are uniform over the wave: a whole block of
    // logits is stored without per-element guards.
    if (cvalid && m0 + 32 <= M) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        e.logits[(int64_t)(m0 + acc_row(r, g)) * e.V + col] = acc[r];
    } else if (cvalid) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + acc_row(r, g);
        if (row < M) e.logits[(int64_t)row * e.V + col] = acc[r];
      }
    }
  }
  rs_step<16, 8>(m, l, lr);
  rs_step<8, 4>(m, l, lr);
  rs_step<4, 2>(m, l, lr);
  rs_step<2, 1>(m, l, lr);
  lse_merge(m[0], l[0], swz_xor<1>(m[0]), swz_xor<1>(l[0]));
  const int row = m0 + acc_row((lr >> 1) & 15, g);
  // V is a multiple of 32, so a block is wholly inside or outside the vocabulary.
  if ((lr & 1) == 0 && row < M && cvalid)
    e.part[(int64_t)row * e.nb + (col >> 5)] = make_float2(m[0], l[0]);
}

// dlogit = g (softmax - onehot(t)) of logit v in column n from the base-2
// log-sum-exp; 0 on ignored rows. Shared by the backward epilogue and the
// fused call's kernel, so both produce the same bits.
__device__ __forceinline__ float ce_dlogit(float v, int n, float lse2, float g, int t, int V) {
  const bool valid = t >= 0 && t < V;
  const float q = fast_exp2(fmaf(v, kLog2e, -lse2)) - (n == t ? 1.f : 0.f);
  return valid ? q * g : 0.f;
}

// Backward epilogue: dlogit from the recomputed logit and the forward's
// base-2 log-sum-exp.
template <typename T>
struct EpiCEGrad {
  T* dl; int64_t ldo; const float* lse2; const int* targets; const float* dloss; int V;
  static constexpr bool kPair = false;
  using Out = T;
  static constexpr int kOuts = 1;
  static constexpr bool kStaged = true;
  struct Col {};
  struct Pre { float lse2, g; int t; };
  __device__ __forceinline__ Col col(int) const { return {}; }
  __device__ __forceinline__ Pre pre(int m, int, const Col&) const {
    return {lse2[m], dloss[m], targets[m]};
  }
  __device__ __forceinline__ bool has(int) const { return true; }
  __device__ __forceinline__ bool vec_ok(int vec) const { return al16(dl) && ldo % vec == 0; }
  __device__ __forceinline__ float value(int, int, int n, float v, float, const Col&,
                                         const Pre& p) const {
    return ce_dlogit(v, n, p.lse2, p.g, p.t, V);
  }
  __device__ __forceinline__ Out* dst(int, int m, int n) const { return dl + (int64_t)m * ldo + n; }
};

// Fused call: dlogits [rows, V] of a chunk from its stored fp32 logits. One
// thread per four consecutive columns of a row (V is a multiple of 64).
template <typename T>
__global__ __launch_bounds__(256) void ce_dlogit_kernel(const float* __restrict__ logits,
                                                        const float* __restrict__ lse2,
                                                        const int* __restrict__ targets,
                                                        const float* __restrict__ dloss, int rows,
                                                        int V, T* __restrict__ dl) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int v4 = V / 4;
  if (q >= (int64_t)rows * v4) return;
  const int row = (int)(q / v4), n0 = (int)(q - (int64_t)row * v4) * 4;
  const float l2 = lse2[row], g = dloss[row];
  const int t = targets[row];
  const float4 x = *(const float4*)(logits + (int64_t)row * V + n0);
  T* o = dl + (int64_t)row * V + n0;
  o[0] = from_f32<T>(ce_dlogit(x.x, n0, l2, g, t, V));
  o[1] = from_f32<T>(ce_dlogit(x.y, n0 + 1, l2, g, t, V));
  o[2] = from_f32<T>(ce_dlogit(x.z, n0 + 2, l2, g, t, V));
  o[3] = from_f32<T>(ce_dlogit(x.w, n0 + 3, l2, g, t, V));
}

// Per row: merge the nb partial pairs into the base-2 log-sum-exp (saved for
// the backward) and the loss. One wave per row, four rows per workgroup.
__global__ __launch_bounds__(256) void ce_combine_kernel(const float2* __restrict__ part,
                                                         int64_t nb, const float* __restrict__ tlogit,
                                                         const int* __restrict__ targets, int rows,
                                                         int V, float* __restrict__ lse2,
                                                         float* __restrict__ loss) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  float m = -INFINITY, l = 0.f;
  const float2* p = part + (int64_t)row * nb;
  for (int64_t j = lane; j < nb; j += 64) {
    const float2 v = p[j];
    lse_merge(m, l, v.x, v.y);
  }
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) {
    const float m2 = __shfl_xor(m, k, 64), l2 = __shfl_xor(l, k, 64);
    lse_merge(m, l, m2, l2);
  }
  if (lane == 0) {
    const int t = targets[row];
    const float L2 = m + __log2f(l);
    lse2[row] = L2;
    loss[row] = (t >= 0 && t < V) ? L2 * kLn2 - tlogit[row] : 0.f;
  }
}

}  // namespace bpt
