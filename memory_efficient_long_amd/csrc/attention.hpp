// Blockwise causal attention on gfx950: forward with an online softmax and a
// recompute-based backward.
//
// Forward ("Blockwise Parallel Transformer for Long Context Large Models",
// §3.4: blockwise attention with renormalisation, Algorithm 1): a workgroup
// owns 128 query rows of one head (32 per wave) and streams 64-row key/value
// tiles through LDS. Each wave computes S^T = K Q^T for its rows, so every lane
// holds whole score columns of ONE query row: the running max, the running
// denominator and the rescale of the output accumulator are lane-local (one
// cross-half exchange per tile). P is rounded to the storage type and fed
// straight from registers into O^T += V^T P^T. Causal masking compares key and
// query indices on the diagonal tiles only. Output: O (token-major) and a
// base-2 log-sum-exp per (head, row).
//
// Backward ("Training memory: model states, activations and checkpointing",
// §2 softmax rule dz = p * (pbar - <p, pbar>) and §3 FlashAttention's saved
// set): a workgroup owns 128 key/value rows of one KV head (32 per wave, kept
// in registers) and walks the query tiles at or after its diagonal for every
// query head of its GQA group. Per 64-row query tile it recomputes S, forms
// P = exp2(S * log2(e) / sqrt(d) - lse), dP = dO V^T, dS = P (dP - D) with
// D = rowsum(dO * O), accumulates dV += P^T dO and dK += dS^T Q in registers,
// and adds dQ = dS K into an fp32 buffer with atomics.
#pragma once

#include "device_common.hpp"

namespace bpt {

template <typename T>
struct AttnFwdArgs {
  const T* q; const T* k; const T* v;  // head-major: q [nh, s, D], k/v [nkv, s, D]
  T* o; int64_t ldo;                    // token-major; head hq at column hq * D
  float* lse;                           // [nh, s], base 2
  int s, nh, group, causal;
  float scale_log2;                     // log2(e) / sqrt(D)
};

template <typename T>
struct AttnBwdArgs {
  const T* q; const T* k; const T* v;   // head-major, as in the forward
  const T* dout; int64_t lddo;          // token-major, head hq at column hq * D
  const float* lse; const float* dvec;  // [nh, s]
  float* dq; int64_t lddq;              // fp32 accumulator, token-major, head hq at hq * D
  T* dk; T* dv; int64_t lddkv;          // token-major, KV head hk at column hk * D
  const float2* rope;                   // cos/sin [s, D/2] or null
  int s, nh, nkv, group, causal;
  float scale_log2, scale;              // log2(e)/sqrt(D), 1/sqrt(D)
};

// Map a workgroup id to (head, tile). Workgroups are dealt round-robin to the
// 8 XCDs; when the head count allows, each XCD gets whole heads so the
// workgroups resident on it stream the same K/V (or Q/dO) tiles through its L2.
// "reverse" orders tiles from the last (longest causal range) to the first.
__device__ __forceinline__ void map_head_tile(int bid, int nheads, int ntiles, bool reverse,
                                              int& head, int& tile) {
  int j;
  if ((nheads & 7) == 0) {
    const int xcd = bid & 7, local = bid >> 3, hpx = nheads >> 3;
    head = xcd * hpx + local % hpx;
    j = local / hpx;
  } else {
    head = bid % nheads;
    j = bid / nheads;
  }
  tile = reverse ? ntiles - 1 - j : j;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_fwd_kernel(AttnFwdArgs<T> a) {
  constexpr int BQ = 128, BKV = 64;
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int LDK = D + VEC;                          // K tile row (16 B pad)
  constexpr int LDV = BKV + (sizeof(T) == 2 ? 4 : 4);   // V^T tile row (8 B / 16 B pad)
  constexpr int NC = D / 16;                            // reduction chunks over d
  constexpr int ND = D / 32;                            // 32-wide d blocks
  __shared__ __attribute__((aligned(16))) T ks[2][BKV * LDK];
  __shared__ __attribute__((aligned(16))) T vt[2][D * LDV];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, g = lane >> 5;
  const int s = a.s;
  const int nqt = (s + BQ - 1) / BQ;
  int hq, qt;
  map_head_tile(blockIdx.x, a.nh, nqt, a.causal != 0, hq, qt);
  const int hk = hq / a.group;
  const int q0 = qt * BQ;
  const int qrow = q0 + 32 * w + lr;
  const T* Qp = a.q + (int64_t)hq * s * D;
  const T* Kp = a.k + (int64_t)hk * s * D;
  const T* Vp = a.v + (int64_t)hk * s * D;

  typename Frag<T>::type qf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (qrow < s) qf[c] = ld_frag(Qp + (int64_t)qrow * D + 16 * c + 8 * g);
    else {
      float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      qf[c] = pack_frag<T>(z);
    }
  }

  const int kv_end = a.causal ? min(s, q0 + BQ) : s;
  const int ntiles = (kv_end + BKV - 1) / BKV;
  const bool wave_active = q0 + 32 * w < s;
  const int wave_last = min(q0 + 32 * w + 31, s - 1);
  const int wave_tiles = a.causal ? wave_last / BKV + 1 : ntiles;

  // K tile: 64 x D, K-contiguous rows; V tile stored transposed (V^T, D x 64).
  constexpr int KCH = BKV * D / VEC / 256;              // 16-byte loads per thread
  constexpr int VSB = (BKV / 4) * (D / VEC);            // 4 x VEC sub-blocks
  constexpr int VCH = (VSB + 255) / 256;
  u32x4 kreg[KCH], vreg[VCH][4];

  auto load_tile = [&](int t) {
    const int kv0 = t * BKV;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i;
      const int r = c / (D / VEC), dc = (c % (D / VEC)) * VEC;
      kreg[i] = (kv0 + r < s) ? ld<u32x4>(Kp + (int64_t)(kv0 + r) * D + dc) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int sb = tid + 256 * i;
      const int kb = sb % (BKV / 4), db = sb / (BKV / 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kv = kv0 + 4 * kb + j;
        vreg[i][j] = (sb < VSB && kv < s) ? ld<u32x4>(Vp + (int64_t)kv * D + db * VEC)
                                          : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i;
      const int r = c / (D / VEC), dc = (c % (D / VEC)) * VEC;
      st<u32x4>(&ks[buf][r * LDK + dc], kreg[i]);
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int sb = tid + 256 * i;
      if (sb < VSB) {
        const int kb = sb % (BKV / 4), db = sb / (BKV / 4);
        if constexpr (sizeof(T) == 2) {
          u32x2 out[8];
          transpose_4xvec(vreg[i], out);
#pragma unroll
          for (int j = 0; j < 8; ++j) st<u32x2>(&vt[buf][(db * 8 + j) * LDV + 4 * kb], out[j]);
        } else {
          u32x4 out[4];
          transpose_4xvec(vreg[i], out);
#pragma unroll
          for (int j = 0; j < 4; ++j) st<u32x4>(&vt[buf][(db * 4 + j) * LDV + 4 * kb], out[j]);
        }
      }
    }
  };

  f32x16 oacc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) oacc[i] = zero16();
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale_log2;

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    if (wave_active && t < wave_tiles) {
      f32x16 sacc[2] = {zero16(), zero16()};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          auto kf = ld_frag(&ks[buf][(32 * sb + lr) * LDK + 16 * c + 8 * g]);
          sacc[sb] = mma(kf, qf[c], sacc[sb]);
        }
      }
      const int kvb = t * BKV;
      const bool need_mask = a.causal ? (kvb + BKV - 1 > q0 + 32 * w) : (kvb + BKV > s);
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = sacc[sb][r];
          if (need_mask) {
            const int kv = kvb + 32 * sb + acc_row(r, g);
            if (kv >= s || (a.causal && kv > qrow)) v = -INFINITY;
          }
          sacc[sb][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * sl2);
      const float alpha = fast_exp2(m_run - m_new);
      float rs = 0.f;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(fmaf(sacc[sb][r], sl2, -m_new));
          sacc[sb][r] = p;
          rs += p;
        }
      rs += shfl_xor(rs, 32);
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
      // P fragments: chunk cc covers keys 16cc + {8(e/4) + 4g + e%4}.
      typename Frag<T>::type pf[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        float tmp[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) tmp[e] = sacc[cc >> 1][8 * (cc & 1) + e];
        pf[cc] = pack_frag<T>(tmp);
      }
#pragma unroll
      for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const T* row = &vt[buf][(32 * i + lr) * LDV + 16 * cc + 4 * g];
          auto vf = ld_frag_split(row, row + 8);
          oacc[i] = mma(vf, pf[cc], oacc[i]);
        }
    }
    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (wave_active && qrow < s) {
    const float inv_l = 1.f / l_run;
    T* orow = a.o + (int64_t)qrow * a.ldo + (int64_t)hq * D;
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * i + r4 * 8 + 4 * g;
#pragma unroll
        for (int e = 0; e < 4; ++e) orow[d + e] = from_f32<T>(oacc[i][4 * r4 + e] * inv_l);
      }
    if (g == 0) a.lse[(int64_t)hq * s + qrow] = m_run + __log2f(l_run);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_kernel(AttnBwdArgs<T> a) {
  constexpr int BQ = 64, BKV = 128;
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int LDR = D + VEC;                            // Q/dO rows (K-contiguous)
  constexpr int LDT = BQ + (sizeof(T) == 2 ? 4 : 4);      // Q^T/dO^T rows
  constexpr int LDKT = BKV + VEC;                         // K^T rows
  constexpr int LDS_ = BKV + VEC;                         // dS rows
  constexpr int NC = D / 16, ND = D / 32;
  __shared__ __attribute__((aligned(16))) T qs[BQ * LDR];
  __shared__ __attribute__((aligned(16))) T dos[BQ * LDR];
  __shared__ __attribute__((aligned(16))) T qts[D * LDT];
  __shared__ __attribute__((aligned(16))) T dots[D * LDT];
  __shared__ __attribute__((aligned(16))) T kts[D * LDKT];
  __shared__ __attribute__((aligned(16))) T dss[BQ * LDS_];
  __shared__ float lse_s[BQ], dd_s[BQ];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, g = lane >> 5;
  const int s = a.s;
  const int nkt = (s + BKV - 1) / BKV;
  int hk, kt;
  map_head_tile(blockIdx.x, a.nkv, nkt, false, hk, kt);
  const int kv0 = kt * BKV;
  const int kvrow = kv0 + 32 * w + lr;
  const T* Kp = a.k + (int64_t)hk * s * D;
  const T* Vp = a.v + (int64_t)hk * s * D;

  // This wave's 32 key/value rows as B operands (lane = key row).
  typename Frag<T>::type kf[NC], vf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (kvrow < s) {
      kf[c] = ld_frag(Kp + (int64_t)kvrow * D + 16 * c + 8 * g);
      vf[c] = ld_frag(Vp + (int64_t)kvrow * D + 16 * c + 8 * g);
    } else {
      float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      kf[c] = pack_frag<T>(z);
      vf[c] = kf[c];
    }
  }
  // K^T of the workgroup's 128 rows in LDS (B operand of dQ = dS K).
  {
    constexpr int SB = (BKV / 4) * (D / VEC);
    for (int sb = tid; sb < SB; sb += 256) {
      const int kb = sb % (BKV / 4), db = sb / (BKV / 4);
      u32x4 in[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kv = kv0 + 4 * kb + j;
        in[j] = kv < s ? ld<u32x4>(Kp + (int64_t)kv * D + db * VEC) : u32x4{0u, 0u, 0u, 0u};
      }
      if constexpr (sizeof(T) == 2) {
        u32x2 out[8];
        transpose_4xvec(in, out);
#pragma unroll
        for (int j = 0; j < 8; ++j) st<u32x2>(&kts[(db * 8 + j) * LDKT + 4 * kb], out[j]);
      } else {
        u32x4 out[4];
        transpose_4xvec(in, out);
#pragma unroll
        for (int j = 0; j < 4; ++j) st<u32x4>(&kts[(db * 4 + j) * LDKT + 4 * kb], out[j]);
      }
    }
  }

  f32x16 dkacc[ND], dvacc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) { dkacc[i] = zero16(); dvacc[i] = zero16(); }

  const float sl2 = a.scale_log2;
  const int nqt = (s + BQ - 1) / BQ;
  const int qt0 = a.causal ? kv0 / BQ : 0;

  for (int gi = 0; gi < a.group; ++gi) {
    const int hq = hk * a.group + gi;
    const T* Qp = a.q + (int64_t)hq * s * D;
    const T* dOp = a.dout + (int64_t)hq * D;
    const float* lsep = a.lse + (int64_t)hq * s;
    const float* dvp = a.dvec + (int64_t)hq * s;
    for (int qt = qt0; qt < nqt; ++qt) {
      const int q0 = qt * BQ;
      __syncthreads();
      // Q and dO tiles, both row-major and transposed.
      {
        constexpr int SB = (BQ / 4) * (D / VEC);
        for (int sb = tid; sb < SB; sb += 256) {
          const int qb = sb % (BQ / 4), db = sb / (BQ / 4);
          u32x4 qin[4], din[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int qr = q0 + 4 * qb + j;
            const bool ok = qr < s;
            qin[j] = ok ? ld<u32x4>(Qp + (int64_t)qr * D + db * VEC) : u32x4{0u, 0u, 0u, 0u};
            din[j] = ok ? ld<u32x4>(dOp + (int64_t)qr * a.lddo + db * VEC) : u32x4{0u, 0u, 0u, 0u};
            st<u32x4>(&qs[(4 * qb + j) * LDR + db * VEC], qin[j]);
            st<u32x4>(&dos[(4 * qb + j) * LDR + db * VEC], din[j]);
          }
          if constexpr (sizeof(T) == 2) {
            u32x2 out[8];
            transpose_4xvec(qin, out);
#pragma unroll
            for (int j = 0; j < 8; ++j) st<u32x2>(&qts[(db * 8 + j) * LDT + 4 * qb], out[j]);
            transpose_4xvec(din, out);
#pragma unroll
            for (int j = 0; j < 8; ++j) st<u32x2>(&dots[(db * 8 + j) * LDT + 4 * qb], out[j]);
          } else {
            u32x4 out[4];
            transpose_4xvec(qin, out);
#pragma unroll
            for (int j = 0; j < 4; ++j) st<u32x4>(&qts[(db * 4 + j) * LDT + 4 * qb], out[j]);
            transpose_4xvec(din, out);
#pragma unroll
            for (int j = 0; j < 4; ++j) st<u32x4>(&dots[(db * 4 + j) * LDT + 4 * qb], out[j]);
          }
        }
        if (tid < BQ) {
          const int qr = q0 + tid;
          lse_s[tid] = qr < s ? lsep[qr] : INFINITY;
          dd_s[tid] = qr < s ? dvp[qr] : 0.f;
        }
      }
      __syncthreads();

      // S = Q K^T and dP = dO V^T for this wave's 32 keys (lane = key).
      f32x16 pr[2], dsr[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          auto qa = ld_frag(&qs[(32 * qb + lr) * LDR + 16 * c + 8 * g]);
          sacc = mma(qa, kf[c], sacc);
          auto da = ld_frag(&dos[(32 * qb + lr) * LDR + 16 * c + 8 * g]);
          dpacc = mma(da, vf[c], dpacc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = 32 * qb + acc_row(r, g);
          const int qg = q0 + ql;
          float p = fast_exp2(fmaf(sacc[r], sl2, -lse_s[ql]));
          if (kvrow >= s || (a.causal && kvrow > qg)) p = 0.f;
          pr[qb][r] = p;
          dsr[qb][r] = p * (dpacc[r] - dd_s[ql]);
        }
      }
      // dV += P^T dO, dK += dS^T Q (A operands straight from registers).
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        float tp[8], td[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          tp[e] = pr[cc >> 1][8 * (cc & 1) + e];
          td[e] = dsr[cc >> 1][8 * (cc & 1) + e];
        }
        auto pa = pack_frag<T>(tp);
        auto dsa = pack_frag<T>(td);
#pragma unroll
        for (int i = 0; i < ND; ++i) {
          const T* dor = &dots[(32 * i + lr) * LDT + 16 * cc + 4 * g];
          dvacc[i] = mma(pa, ld_frag_split(dor, dor + 8), dvacc[i]);
          const T* qr = &qts[(32 * i + lr) * LDT + 16 * cc + 4 * g];
          dkacc[i] = mma(dsa, ld_frag_split(qr, qr + 8), dkacc[i]);
        }
      }
      // dS to LDS, [query][key], for dQ = dS K.
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          dss[(32 * qb + acc_row(r, g)) * LDS_ + 32 * w + lr] = from_f32<T>(dsr[qb][r]);
      __syncthreads();

      // dQ tile (64 x D) split over the 4 waves: query block w & 1.
      {
        constexpr int NB = ND >= 2 ? ND / 2 : 1;
        const int qb = w & 1;
        const bool active = ND >= 2 || w < 2;
#pragma unroll
        for (int bi = 0; bi < NB; ++bi) {
          const int db = ND >= 2 ? (w >> 1) * NB + bi : 0;
          if (active) {
            f32x16 acc = zero16();
#pragma unroll
            for (int kk = 0; kk < BKV / 16; ++kk) {
              auto sa = ld_frag(&dss[(32 * qb + lr) * LDS_ + 16 * kk + 8 * g]);
              auto kb = ld_frag(&kts[(32 * db + lr) * LDKT + 16 * kk + 8 * g]);
              acc = mma(sa, kb, acc);
            }
            float* dqp = a.dq + (int64_t)hq * D + 32 * db + lr;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int qg = q0 + 32 * qb + acc_row(r, g);
              if (qg < s) atomicAdd(dqp + (int64_t)qg * a.lddq, acc[r] * a.scale);
            }
          }
        }
      }
    }
  }

  // dK (scaled, RoPE inverse) and dV to the token-major outputs.
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    const int d = 32 * i + lr;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kv = kv0 + 32 * w + acc_row(r, g);
      float dkv = dkacc[i][r] * a.scale;
      float pair = shfl_xor(dkv, 1);
      if (a.rope && kv < s) {
        float2 cs = a.rope[(int64_t)kv * (D / 2) + (d >> 1)];
        // inverse rotation: [c s; -s c]
        dkv = (d & 1) ? (dkv * cs.x - pair * cs.y) : (dkv * cs.x + pair * cs.y);
      }
      if (kv < s) {
        a.dk[(int64_t)kv * a.lddkv + (int64_t)hk * D + d] = from_f32<T>(dkv);
        a.dv[(int64_t)kv * a.lddkv + (int64_t)hk * D + d] = from_f32<T>(dvacc[i][r]);
      }
    }
  }
}

}  // namespace bpt
