// Row-wise and reduction kernels of the layer: LayerNorm / RMSNorm forward and
// backward (one wave per row, statistics in fp32), column sums for bias and
// norm-parameter gradients (deterministic two-stage), the RoPE cos/sin table,
// and the attention-backward row term D = rowsum(dO * O).
#pragma once

#include "device_common.hpp"

namespace bpt {

__device__ __forceinline__ void load8(const bf16* p, float v[8]) {
  bf16x8 x = ld<bf16x8>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
}
__device__ __forceinline__ void load8(const float* p, float v[8]) {
  f32x4 a = ld<f32x4>(p), b = ld<f32x4>(p + 4);
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
}
__device__ __forceinline__ void store8(bf16* p, const float v[8]) {
  bf16x8 x;
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (bf16)v[e];
  st<bf16x8>(p, x);
}
__device__ __forceinline__ void store8(float* p, const float v[8]) {
  st<f32x4>(p, f32x4{v[0], v[1], v[2], v[3]});
  st<f32x4>(p + 4, f32x4{v[4], v[5], v[6], v[7]});
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}

enum NormKind { NORM_LAYER = 0, NORM_RMS = 1 };

// out = Norm(x) * gamma (+ beta). NCH: 8-element chunks per lane (h <= 512 * NCH).
template <typename T, typename Tin, typename Tout, int NCH>
__global__ __launch_bounds__(256) void norm_fwd_kernel(const Tin* __restrict__ x, int64_t ldx,
                                                       const T* __restrict__ gamma,
                                                       const T* __restrict__ beta, Tout* out,
                                                       int64_t ldo, int rows, int h, int kind,
                                                       float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int nch = h / 8;
  float v[NCH][8];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      load8(x + (int64_t)row * ldx + 8 * c, v[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += v[i][e];
    }
  }
  const float inv_h = 1.f / (float)h;
  float mean = 0.f;
  if (kind == NORM_LAYER) mean = wave_sum(sum) * inv_h;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i)
    if (lane + 64 * i < nch)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = v[i][e] - mean;
        sq += d * d;
      }
  const float rstd = 1.f / sqrtf(wave_sum(sq) * inv_h + eps);
  // gamma / beta need only element alignment; 16-byte aligned ones (the
  // usual case, a uniform test) are read as vectors.
  const bool gvec = (((uintptr_t)gamma | (uintptr_t)beta) & 15) == 0;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      float gm[8], bt[8], o[8];
      if (gvec) {
        load8(gamma + 8 * c, gm);
        if (beta) load8(beta + 8 * c, bt);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          gm[e] = to_f32(gamma[8 * c + e]);
          if (beta) bt[e] = to_f32(beta[8 * c + e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float y = (v[i][e] - mean) * rstd * gm[e];
        if (beta) y += bt[e];
        o[e] = y;
      }
      store8(out + (int64_t)row * ldo + 8 * c, o);
    }
  }
}

// Norm backward fused with the residual:
//   out = res + rstd * (gx - [mean(gx)] - xhat * mean(gx * xhat)),  gx = dz * gamma
// (the bracketed term only for LayerNorm). A row is handled by WPR waves (one,
// or all four of the workgroup for wide rows, so that a lane holds at most
// 8 NCH elements of each per-row array and nothing spills); rows are strided
// over these units. Each unit keeps fp32 partial sums of dz * xhat and dz for
// the scale and shift gradients and writes them to part_g / part_b [units, h].
template <typename T, typename Tin, typename Tres, int NCH, int WPR>
__global__ __launch_bounds__(256) void norm_bwd_kernel(
    const float* __restrict__ dz, int64_t lddz, const Tin* __restrict__ xin, int64_t ldx,
    const T* __restrict__ gamma, const Tres* __restrict__ res, int64_t ldr, float* out_f,
    T* out_t, int64_t ldo, float* part_g, float* part_b, int rows, int h, int kind, float eps,
    int accumulate_part) {
  static_assert(WPR == 1 || WPR == 4, "waves per row");
  constexpr int CW = 64 * WPR;  // chunk stride of a unit
  const int lane = (WPR == 1 ? threadIdx.x & 63 : threadIdx.x);
  const int wid = threadIdx.x >> 6;
  const int wave = WPR == 1 ? blockIdx.x * 4 + wid : blockIdx.x;  // unit index
  const int nwaves = WPR == 1 ? gridDim.x * 4 : gridDim.x;
  const int nch = h / 8;
  __shared__ float red[2][4];
  // Sum over the unit (two values at once); WPR = 4 exchanges the per-wave
  // sums through LDS, with barriers on both sides so the slots can be reused.
  auto unit_sum2 = [&](float& a, float& b) {
    a = wave_sum(a);
    b = wave_sum(b);
    if constexpr (WPR == 4) {
      if ((threadIdx.x & 63) == 0) { red[0][wid] = a; red[1][wid] = b; }
      __syncthreads();
      a = red[0][0] + red[0][1] + red[0][2] + red[0][3];
      b = red[1][0] + red[1][1] + red[1][2] + red[1][3];
      __syncthreads();
    }
  };
  const float inv_h = 1.f / (float)h;
  const bool gvec = ((uintptr_t)gamma & 15) == 0;  // uniform: vector reads of gamma
  float pg[NCH][8], pb[NCH][8];
#pragma unroll
  for (int i = 0; i < NCH; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) { pg[i][e] = 0.f; pb[i][e] = 0.f; }

  for (int row = wave; row < rows; row += nwaves) {
    float xv[NCH][8], gv[NCH][8];
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + CW * i;
      if (c < nch) {
        load8(xin + (int64_t)row * ldx + 8 * c, xv[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += xv[i][e];
      }
    }
    float mean = 0.f, dummy = 0.f;
    if (kind == NORM_LAYER) {
      unit_sum2(sum, dummy);
      mean = sum * inv_h;
    }
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      if (lane + CW * i < nch)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = xv[i][e] - mean;
          sq += d * d;
        }
    unit_sum2(sq, dummy);
    const float rstd = 1.f / sqrtf(sq * inv_h + eps);
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + CW * i;
      if (c < nch) {
        float dzv[8], gm[8];
        load8(dz + (int64_t)row * lddz + 8 * c, dzv);
        if (gvec) {
          load8(gamma + 8 * c, gm);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) gm[e] = to_f32(gamma[8 * c + e]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xh = (xv[i][e] - mean) * rstd;
          xv[i][e] = xh;
          const float gx = dzv[e] * gm[e];
          gv[i][e] = gx;
          s1 += gx;
          s2 += gx * xh;
          pg[i][e] += dzv[e] * xh;
          pb[i][e] += dzv[e];
        }
      }
    }
    unit_sum2(s1, s2);
    const float m1 = kind == NORM_LAYER ? s1 * inv_h : 0.f;
    const float m2 = s2 * inv_h;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + CW * i;
      if (c < nch) {
        float rv[8], o[8];
        load8(res + (int64_t)row * ldr + 8 * c, rv);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = rv[e] + rstd * (gv[i][e] - m1 - xv[i][e] * m2);
        if (out_f) store8(out_f + (int64_t)row * ldo + 8 * c, o);
        if (out_t) store8(out_t + (int64_t)row * ldo + 8 * c, o);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + CW * i;
    if (c < nch) {
      if (accumulate_part) {  // running partials over several calls
        float og[8], ob[8];
        if (part_g) {
          load8(part_g + (int64_t)wave * h + 8 * c, og);
#pragma unroll
          for (int e = 0; e < 8; ++e) pg[i][e] += og[e];
        }
        if (part_b) {
          load8(part_b + (int64_t)wave * h + 8 * c, ob);
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[i][e] += ob[e];
        }
      }
      if (part_g) store8(part_g + (int64_t)wave * h + 8 * c, pg[i]);
      if (part_b) store8(part_b + (int64_t)wave * h + 8 * c, pb[i]);
    }
  }
}

// Stage 1 of a column sum over X [rows, N]: grid (ceil(N / 64), P); block
// (64 columns x 4 row lanes); part[blockIdx.y, col] = sum over the block's rows.
template <typename Tin>
__global__ __launch_bounds__(256) void colsum_partial_kernel(const Tin* __restrict__ X, int64_t ldx,
                                                             int rows, int N, float* part,
                                                             int accumulate) {
  __shared__ float red[4][64];
  const int cl = threadIdx.x & 63, rl = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + cl;
  const int per = (rows + gridDim.y - 1) / gridDim.y;
  const int r0 = blockIdx.y * per, r1 = min(rows, r0 + per);
  float acc = 0.f;
  if (col < N)
    for (int r = r0 + rl; r < r1; r += 4) acc += to_f32(X[(int64_t)r * ldx + col]);
  red[rl][cl] = acc;
  __syncthreads();
  if (rl == 0 && col < N) {
    const float v = red[0][cl] + red[1][cl] + red[2][cl] + red[3][cl];
    float* o = part + (int64_t)blockIdx.y * N + col;
    *o = accumulate ? *o + v : v;
  }
}

// Stage 1 with 16-byte loads (X 16-byte aligned, N and ldx multiples of the
// vector width V): each thread sums V adjacent columns, so a wave reads 1 KiB
// of a row per load; rows are taken four at a time per lane to keep several
// loads in flight. Same grid semantics as above with 64 V columns per block.
template <typename Tin>
__global__ __launch_bounds__(256) void colsum_partial_vec_kernel(const Tin* __restrict__ X,
                                                                 int64_t ldx, int rows, int N,
                                                                 float* part, int accumulate) {
  constexpr int V = 16 / (int)sizeof(Tin);
  struct Elems { Tin e[V]; };
  __shared__ float red[4][64 * V];
  const int cl = threadIdx.x & 63, rl = threadIdx.x >> 6;
  const int c0 = (blockIdx.x * 64 + cl) * V;
  const int per = (rows + gridDim.y - 1) / gridDim.y;
  const int r0 = blockIdx.y * per, r1 = min(rows, r0 + per);
  float acc[V];
#pragma unroll
  for (int j = 0; j < V; ++j) acc[j] = 0.f;
  if (c0 < N) {
    const Tin* base = X + c0;
    int r = r0 + rl;
    for (; r + 12 < r1; r += 16) {
      u32x4 u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) u[i] = *(const u32x4*)(base + (int64_t)(r + 4 * i) * ldx);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const Elems x = __builtin_bit_cast(Elems, u[i]);
#pragma unroll
        for (int j = 0; j < V; ++j) acc[j] += to_f32(x.e[j]);
      }
    }
    for (; r < r1; r += 4) {
      const Elems x = __builtin_bit_cast(Elems, *(const u32x4*)(base + (int64_t)r * ldx));
#pragma unroll
      for (int j = 0; j < V; ++j) acc[j] += to_f32(x.e[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < V; ++j) red[rl][cl * V + j] = acc[j];
  __syncthreads();
  for (int c = threadIdx.x; c < 64 * V; c += 256) {
    const int col = blockIdx.x * 64 * V + c;
    if (col < N) {
      const float v = red[0][c] + red[1][c] + red[2][c] + red[3][c];
      float* o = part + (int64_t)blockIdx.y * N + col;
      *o = accumulate ? *o + v : v;
    }
  }
}

// Stage 2: out[col] (+)= sum_p part[p, col]; block = 64 columns x 16
// partial lanes (1024 threads), each lane summing every 16th partial row with
// up to 16 of its loads in flight at a time, then an LDS reduction. (With 4
// lanes per column and its loads waited for one by one, the reduction of the
// norm backward's 2048 partial rows took ~40-60 us per call on 32 blocks.)
constexpr int kColsumFinalLanes = 16;
__global__ __launch_bounds__(64 * kColsumFinalLanes) void colsum_final_kernel(
    const float* __restrict__ part, int P, int N, float* out, int accumulate) {
  constexpr int L = kColsumFinalLanes, U = 16;
  __shared__ float red[L][64];
  const int cl = threadIdx.x & 63, rl = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + cl;
  float a = 0.f;
  if (col < N) {
    for (int p0 = rl; p0 < P; p0 += L * U) {
      float v[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int p = p0 + L * i;
        v[i] = p < P ? part[(int64_t)p * N + col] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < U; ++i) a += v[i];
    }
  }
  red[rl][cl] = a;
  __syncthreads();
  if (rl == 0 && col < N) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < L; ++j) acc += red[j][cl];
    out[col] = accumulate ? out[col] + acc : acc;
  }
}

// dst[r, j] = src[r, off_k + (j - start_k)] for the three column segments
// [0, c1), [c1, c2), [c2, n) of dst (start_k = 0, c1, c2): gathers a head
// chunk's Q, K and V columns of the packed projection into one contiguous
// block. One thread copies V elements (V = 1, or 16 bytes when the source
// rows and every width and offset are 16-byte multiples).
template <typename T, int V>
__global__ __launch_bounds__(256) void gather_cols3_kernel(const T* __restrict__ src, int64_t lds,
                                                           T* __restrict__ dst, int rows, int c1,
                                                           int c2, int n, int64_t off0,
                                                           int64_t off1, int64_t off2) {
  struct Vec { T e[V]; };
  const int vpr = n / V;  // vectors per row
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)rows * vpr) return;
  const int r = (int)(i / vpr), j = (int)(i - (int64_t)r * vpr) * V;
  const int64_t sc = j < c1 ? off0 + j : (j < c2 ? off1 + (j - c1) : off2 + (j - c2));
  *(Vec*)(dst + (int64_t)r * n + j) = *(const Vec*)(src + (int64_t)r * lds + sc);
}

__global__ __launch_bounds__(256) void fill_kernel(float* p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// RoPE table: tab[p, i] = (cos, sin)(p * base^(-2i/D)), angles in fp64.
__global__ __launch_bounds__(256) void rope_table_kernel(float2* tab, int s, int D, double base) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int half = D / 2;
  if (idx >= (int64_t)s * half) return;
  const int p = (int)(idx / half), i = (int)(idx % half);
  const double theta = pow(base, -2.0 * (double)i / (double)D);
  const double ang = (double)p * theta;
  tab[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

// D[h, q] = sum_d dO[q, h D + d] * O[q, h D + d] (fp32). The L = D / 8 lanes
// of one (row, head) pair each read an 8-element piece, side by side, so a
// wave reads 64 / L consecutive pairs of a row as one contiguous span; the
// pieces are then summed across the L lanes with xor shuffles.
template <typename T, int L>
__global__ __launch_bounds__(256) void attn_dvec_kernel(const T* __restrict__ dout,
                                                        const T* __restrict__ o, int64_t ld,
                                                        float* dvec, int s, int nh) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pair = t / L;
  const int piece = (int)(t % L);
  const bool ok = pair < (int64_t)s * nh;
  int row = 0, h = 0;
  float acc = 0.f;
  if (ok) {
    row = (int)(pair / nh);
    h = (int)(pair - (int64_t)row * nh);
    const int64_t off = (int64_t)row * ld + (int64_t)h * (8 * L) + 8 * piece;
    float va[8], vb[8];
    load8(dout + off, va);
    load8(o + off, vb);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += va[e] * vb[e];
  }
#pragma unroll
  for (int m = L / 2; m >= 1; m >>= 1) acc += shfl_xor(acc, m);
  if (ok && piece == 0) dvec[(int64_t)h * s + row] = acc;
}

}  // namespace bpt
