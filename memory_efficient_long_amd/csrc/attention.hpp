// Blockwise causal attention on gfx950: forward with an online softmax and a
// recompute-based backward split into a dK/dV pass and a dQ pass.
//
// Forward ("Blockwise Parallel Transformer for Long Context Large Models",
// §3.4: blockwise attention with renormalisation, Algorithm 1): a workgroup
// owns 128 query rows of one head (32 per wave) and streams 64-row key/value
// tiles through LDS. Each wave computes S^T = K Q^T for its rows, so every lane
// holds whole score columns of ONE query row: the running max, the running
// denominator and the rescale of the output accumulator are lane-local (one
// cross-half exchange per tile). The running max is only moved when a tile's
// max exceeds it by more than 2^8 (shift invariance of the softmax keeps the
// result exact; exp2 arguments stay <= 8), so the output accumulator is
// rescaled rarely. P is rounded to the storage type and fed straight from
// registers into O^T += V^T P^T. Output: O (token-major) and a base-2
// log-sum-exp per (head, row).
//
// Backward ("Training memory: model states, activations and checkpointing",
// §2 softmax rule dz = p * (pbar - <p, pbar>), and §3 FlashAttention's saved
// set: O plus the per-row log-sum-exp, scores rebuilt in the backward):
//  * dK/dV pass: a workgroup owns 128 key rows of one KV head (32 per wave,
//    held in registers) and walks the query tiles at or after its diagonal for
//    every query head of its GQA group; per 64-row query tile it rebuilds
//    P = exp2(S - lse), dP = dO V^T, dS = P (dP - D) with
//    D = rowsum(dO * O), and accumulates dV += P^T dO, dK += dS^T Q.
//  * dQ pass: a workgroup owns 128 query rows (32 per wave, Q and dO in
//    registers) and streams key/value tiles like the forward, rebuilding P and
//    dS per tile (lane-local row terms) and accumulating dQ^T += K^T dS^T.
// Neither pass needs atomics; the inverse RoPE rotation and the scale factor
// are applied when dQ and dK are written.
//
// Q arrives multiplied by log2(e)/sqrt(d) (the projection's epilogue applies
// it before rounding), so S = Q K^T is already the scaled score in base-2
// units and no kernel scales scores element by element; dK = dS^T q / sqrt(d)
// becomes ln(2) dS^T Q.
#pragma once

#include <type_traits>

#include "device_common.hpp"

namespace bpt {

// ----------------------------------------------------------------- dropout masks
// Dropout on the attention probabilities with masks regenerated from a
// counter-based generator in every pass (nothing is stored): Philox4x32 with
// ten rounds (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC'11). Element (query i, key j) of global query head h in
// sequence b takes byte j % 4 of word i % 4 of the output for the counter
// (i / 4, j / 4, h, b) under the key (seed low, seed high); it is kept iff the
// byte is >= thr. One call serves a 4 x 4 block of (query, key) pairs: a lane
// that owns a query row reads one word (four consecutive keys), a lane that
// owns a key reads one byte of each word (four consecutive queries).
struct Philox4 { uint32_t w[4]; };

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return {{c0, c1, c2, c3}};
}

struct DropArgs {
  uint32_t seed_lo, seed_hi;
  int thr;        // keep iff byte >= thr (1..255); 0: no dropout
  float scale;    // 256 / (256 - thr), applied to kept probabilities
  int head0;      // global index of the launch's query head 0 (head chunks)
  int batch;      // sequence index within the batch
};

// Word `sel` (0..3) of the call for the 4 x 4 block (q4, k4) of head hg.
__device__ __forceinline__ uint32_t drop_word(const DropArgs& d, int q4, int k4, int hg, int sel) {
  const Philox4 r = philox4x32_10((uint32_t)q4, (uint32_t)k4, (uint32_t)hg, (uint32_t)d.batch,
                                  d.seed_lo, d.seed_hi);
  return sel == 0 ? r.w[0] : sel == 1 ? r.w[1] : sel == 2 ? r.w[2] : r.w[3];
}

__device__ __forceinline__ bool drop_keep_byte(uint32_t word, int byte, int thr) {
  return (int)((word >> (8 * byte)) & 0xFFu) >= thr;
}

// ---- Sharing one generator call among the four lanes that need it.
// In the head_dim 64/128 kernels the four lanes of a quad (lanes 4k .. 4k+3)
// own four consecutive queries (or keys) of one 4 x 4 block row (column), so
// they need the same calls. Each lane computes a different one and a 4 x 4
// transpose across the quad redistributes the words: a quarter of the calls.

// Lane value from lane (quad_base + PERM[lane % 4]) (DPP quad_perm; every
// source lane is valid, so the move keeps no old value).
template <int CTRL>
__device__ __forceinline__ uint32_t quad_perm(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}

// 4 x 4 transpose of words across a quad: afterwards lane i holds in a[j] what
// lane j held in a[i]. Two exchange stages (partner lane ^ 1, then ^ 2); in
// each, a lane keeps the two words whose index matches its own lane bit and
// takes the partner's other two.
__device__ __forceinline__ void quad_transpose(uint32_t (&a)[4], int lane) {
  const bool odd = lane & 1, hi = lane & 2;
  {
    const uint32_t s0 = odd ? a[0] : a[1], s1 = odd ? a[2] : a[3];
    const uint32_t r0 = quad_perm<0xB1>(s0), r1 = quad_perm<0xB1>(s1);  // [1, 0, 3, 2]
    a[0] = odd ? r0 : a[0];
    a[1] = odd ? a[1] : r0;
    a[2] = odd ? r1 : a[2];
    a[3] = odd ? a[3] : r1;
  }
  {
    const uint32_t s0 = hi ? a[0] : a[2], s1 = hi ? a[1] : a[3];
    const uint32_t r0 = quad_perm<0x4E>(s0), r1 = quad_perm<0x4E>(s1);  // [2, 3, 0, 1]
    a[0] = hi ? r0 : a[0];
    a[1] = hi ? r1 : a[1];
    a[2] = hi ? a[2] : r0;
    a[3] = hi ? a[3] : r1;
  }
}

// Query-row lanes: lane i of a quad (its query q has q % 4 = i) computes the
// call for key group k4[i] and returns, in w[j], word i of the call for key
// group k4[j] -- the four keys of group k4[j] for its own query.
__device__ __forceinline__ void drop_words_rows(const DropArgs& d, int q4, int my_k4, int hg,
                                                int lane, uint32_t (&w)[4]) {
  const Philox4 c = philox4x32_10((uint32_t)q4, (uint32_t)my_k4, (uint32_t)hg, (uint32_t)d.batch,
                                  d.seed_lo, d.seed_hi);
  w[0] = c.w[0]; w[1] = c.w[1]; w[2] = c.w[2]; w[3] = c.w[3];
  quad_transpose(w, lane);
}

// Key-row lanes: lane i of a quad (its key k has k % 4 = i) computes the call
// for query group q4[i]; returns in b[j] the four bytes i of the words of the
// call for query group q4[j] (byte e: query 4 q4[j] + e with this lane's key).
__device__ __forceinline__ void drop_bytes_cols(const DropArgs& d, int my_q4, int k4, int hg,
                                                int lane, uint32_t (&b)[4]) {
  const Philox4 c = philox4x32_10((uint32_t)my_q4, (uint32_t)k4, (uint32_t)hg, (uint32_t)d.batch,
                                  d.seed_lo, d.seed_hi);
  // byte transpose inside the lane: b[t] = byte t of words 0, 1, 2, 3
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t sel = (uint32_t)t | ((uint32_t)(4 + t) << 8) | 0x0C0C0000u;
    const uint32_t x01 = __builtin_amdgcn_perm(c.w[1], c.w[0], sel);
    const uint32_t x23 = __builtin_amdgcn_perm(c.w[3], c.w[2], sel);
    b[t] = __builtin_amdgcn_perm(x23, x01, 0x05040100u);
  }
  quad_transpose(b, lane);
}

template <typename T>
struct AttnFwdArgs {
  const T* q; const T* k; const T* v;  // head-major: q [nh, s, D] (times log2(e)/sqrt(D)), k/v [nkv, s, D]
  T* o; int64_t ldo;                    // token-major; head hq at column hq * D
  float* lse;                           // [nh, s], base 2
  int s, nh, group, causal;
  int window;                           // causal sliding window W (0: none): keys i - W < j <= i
  DropArgs drop;                        // attention dropout (used by the DROP variants)
};

template <typename T>
struct AttnBwdArgs {
  const T* q; const T* k; const T* v;   // head-major, as in the forward
  const T* dout; int64_t lddo;          // token-major, head hq at column hq * D
  const float* lse; const float* dvec;  // [nh, s]
  T* dq; int64_t lddq;                  // token-major, head hq at column hq * D
  T* dk; T* dv; int64_t lddkv;          // token-major, KV head hk at column hk * D
  const float2* rope;                   // cos/sin [s, D/2] or null
  int s, nh, nkv, group, causal;
  int window;                           // as in AttnFwdArgs
  float scale, dk_scale;                // dQ factor 1/sqrt(D); dK factor ln(2) (Q carries log2(e)/sqrt(D))
  DropArgs drop;                        // attention dropout (used by the DROP variants)
  // dK/dV split over the query heads of a KV head (bf16 head_dim 64/128):
  // nparts > 1 runs nparts workgroups per key tile, each over group / nparts
  // of the query heads, writing raw fp32 sums to part [nparts][2][nkv][s][D]
  // (dK then dV) for dkdv_reduce_kernel.
  float* part; int nparts;
};

// Map a workgroup id to (head, tile). Workgroups are dealt round-robin to the
// 8 XCDs; when the head count allows, each XCD gets whole heads and runs them
// one after the other (all tiles of its first head, then the next), so the
// workgroups resident on it stream the same K/V (or Q/dO) tiles through its L2
// (interleaving two heads per XCD measured 1-2 % slower per attention kernel).
// "reverse" orders tiles from the last (longest causal range) to the first.
__device__ __forceinline__ void map_head_tile(int bid, int nheads, int ntiles, bool reverse,
                                              int& head, int& tile) {
  int j;
  if ((nheads & 7) == 0) {
    const int xcd = bid & 7, local = bid >> 3, hpx = nheads >> 3;
    head = xcd * hpx + local / ntiles;
    j = local % ntiles;
  } else {
    head = bid % nheads;
    j = bid / nheads;
  }
  tile = reverse ? ntiles - 1 - j : j;
}

// Row-major LDS tile of R x D elements, rows padded by 16 bytes and stored at
// permuted positions pi(r) = r ^ ((r >> 3) & 7). With the pad, eight
// consecutive rows (one MFMA fragment read) start on distinct banks; the
// permutation also spreads rows 4 apart (the RowTile store pattern) over
// distinct banks. The permutation is per row, so a lane's base address is
// computed once and fragment offsets stay immediates.
template <typename T, int D>
struct Swz {
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int LD = D + VEC;
  __device__ static __forceinline__ int row(int r) { return r ^ ((r >> 3) & 7); }
  __device__ static __forceinline__ int off(int r, int chunk) { return row(r) * LD + chunk * VEC; }
  // Fragment: 8 consecutive elements [k0, k0 + 8) of row r (k0 % 8 == 0).
  __device__ static __forceinline__ typename Frag<T>::type frag(const T* tile, int r, int k0) {
    return ld_frag(tile + row(r) * LD + k0);
  }
};

// A tile of R rows x D columns (storage T, row stride ld) held in registers as
// 4-row x 16-byte sub-blocks, stored to LDS row-major and/or transposed.
// Consecutive threads take consecutive 4-row groups, so the transposed store
// writes consecutive 8-byte (bf16) or 16-byte (fp32) chunks of one LDS row.
template <typename T, int R, int D>
struct RowTile {
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int SB = (R / 4) * (D / VEC);
  static constexpr int PER = (SB + 255) / 256;
  u32x4 reg[PER][4];

  __device__ __forceinline__ void load(const T* src, int64_t ldm, int r0, int rlim, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int sb = tid + 256 * i;
      const int rb = sb % (R / 4), cb = sb / (R / 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = r0 + 4 * rb + j;
        reg[i][j] = (sb < SB && row < rlim) ? ld<u32x4>(src + (int64_t)row * ldm + cb * VEC)
                                            : u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store_swz(T* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int sb = tid + 256 * i;
      if (sb < SB) {
        const int rb = sb % (R / 4), cb = sb / (R / 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) st<u32x4>(lds + Swz<T, D>::off(4 * rb + j, cb), reg[i][j]);
      }
    }
  }
  __device__ __forceinline__ void store_cols(T* lds, int ldl, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int sb = tid + 256 * i;
      if (sb < SB) {
        const int rb = sb % (R / 4), cb = sb / (R / 4);
        if constexpr (sizeof(T) == 2) {
          u32x2 out[8];
          transpose_4xvec(reg[i], out);
#pragma unroll
          for (int j = 0; j < 8; ++j) st<u32x2>(lds + (cb * 8 + j) * ldl + 4 * rb, out[j]);
        } else {
          u32x4 out[4];
          transpose_4xvec(reg[i], out);
#pragma unroll
          for (int j = 0; j < 4; ++j) st<u32x4>(lds + (cb * 4 + j) * ldl + 4 * rb, out[j]);
        }
      }
    }
  }
};

template <typename T>
__device__ __forceinline__ typename Frag<T>::type zero_frag() {
  float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  return pack_frag<T>(z);
}

// Row pitch padding (elements) of the transposed LDS tiles, read as two
// 4-element halves: 8 bytes (bf16) / 16 bytes (fp32).
template <typename T> constexpr int pad_t() { return sizeof(T) == 2 ? 4 : 4; }

// ============================================================================ forward
template <typename T, int D, bool WIN = false, bool DROP = false>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnFwdArgs<T> a) {
  const int win = WIN ? a.window : 0;  // sliding window (compiled out when WIN is false)
  constexpr int BQ = 128, BKV = 64;
  constexpr int LDV = BKV + pad_t<T>();
  constexpr int NC = D / 16, ND = D / 32;
  __shared__ __attribute__((aligned(16))) T ks[2][BKV * (D + 16 / sizeof(T))];
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
  for (int c = 0; c < NC; ++c)
    qf[c] = qrow < s ? ld_frag(Qp + (int64_t)qrow * D + 16 * c + 8 * g) : zero_frag<T>();

  const int kv_end = a.causal ? min(s, q0 + BQ) : s;
  const int ntiles = (kv_end + BKV - 1) / BKV;
  const bool wave_active = q0 + 32 * w < s;
  const int wave_last = min(q0 + 32 * w + 31, s - 1);
  const int wave_tiles = a.causal ? wave_last / BKV + 1 : ntiles;
  // Sliding window: key tiles wholly before every row's window are skipped.
  const int t_lo = win ? max(0, q0 - win + 1) / BKV : 0;
  const int wave_t_lo = win ? max(0, q0 + 32 * w - win + 1) / BKV : 0;

  RowTile<T, BKV, D> kt, vtile;
  f32x16 oacc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) oacc[i] = zero16();
  float m_run = -INFINITY, l_run = 0.f;

  if (ntiles > t_lo) {
    kt.load(Kp, D, t_lo * BKV, s, tid);
    vtile.load(Vp, D, t_lo * BKV, s, tid);
    kt.store_swz(ks[0], tid);
    vtile.store_cols(vt[0], LDV, tid);
  }
  __syncthreads();

  for (int t = t_lo; t < ntiles; ++t) {
    const int buf = (t - t_lo) & 1;
    if (t + 1 < ntiles) {
      kt.load(Kp, D, (t + 1) * BKV, s, tid);
      vtile.load(Vp, D, (t + 1) * BKV, s, tid);
    }
    if (wave_active && t < wave_tiles && t >= wave_t_lo) {
      const int kvb = t * BKV;
      const bool MASK = (a.causal ? (kvb + BKV - 1 > q0 + 32 * w) : (kvb + BKV > s)) ||
                        (win && kvb <= q0 + 32 * w + 31 - win);
      f32x16 sacc[2] = {zero16(), zero16()};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          auto kf = Swz<T, D>::frag(ks[buf], 32 * sb + lr, 16 * c + 8 * g);
          sacc[sb] = mma(kf, qf[c], sacc[sb]);
        }
      }
      if (MASK) {  // wave-uniform; keys past min(query, s - 1), or W or more before it, get -inf
        const int qc = a.causal ? min(qrow, s - 1) : s - 1;
        const int lim = qc - kvb;
        const int lo = win ? qc - win - kvb : -BKV;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 32 * sb + acc_row(r, g);
            sacc[sb][r] = (off > lim || off <= lo) ? -INFINITY : sacc[sb][r];
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[sb][r]);
      mx = fmaxf(mx, shfl_xor(mx, 32));
      // Move the running max only when this tile exceeds it by > 8 (log2 units).
      if (__any(mx > m_run + 8.f)) {
        const float m_new = fmaxf(m_run, mx);
        // The branch is wave-wide: with a window, a row may still have seen no
        // visible key (m_run = m_new = -inf); it keeps its (zero) state.
        const float alpha = win && m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < ND; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
        m_run = m_new;
      }
      // A row whose keys so far are all outside its window keeps m_run = -inf;
      // its masked scores then give exp2(-inf) = 0 rather than exp2(NaN).
      const float m_sub = win && m_run == -INFINITY ? 0.f : m_run;
      float rs = 0.f;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(sacc[sb][r] - m_sub);
          sacc[sb][r] = p;
          rs += p;
        }
      l_run += rs + shfl_xor(rs, 32);
      if constexpr (DROP) {  // the normaliser above is the undropped one
        const int hg = a.drop.head0 + hq;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t wd =
                drop_word(a.drop, qrow >> 2, (kvb + 32 * sb + 8 * j + 4 * g) >> 2, hg, qrow & 3);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sacc[sb][4 * j + e] = drop_keep_byte(wd, e, a.drop.thr) ? sacc[sb][4 * j + e] : 0.f;
          }
      }
      // P fragments: chunk cc covers keys 16cc + {8(e/4) + 4g + e%4}.
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        float tmp[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) tmp[e] = sacc[cc >> 1][8 * (cc & 1) + e];
        const auto pf = pack_frag<T>(tmp);
#pragma unroll
        for (int i = 0; i < ND; ++i) {
          const T* row = &vt[buf][(32 * i + lr) * LDV + 16 * cc + 4 * g];
          oacc[i] = mma(ld_frag_split(row, row + 8), pf, oacc[i]);
        }
      }
    }
    if (t + 1 < ntiles) {
      kt.store_swz(ks[buf ^ 1], tid);
      vtile.store_cols(vt[buf ^ 1], LDV, tid);
    }
    __syncthreads();
  }

  if (wave_active && qrow < s) {
    const float inv_l = (DROP ? a.drop.scale : 1.f) / l_run;
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

// ============================================================================ backward: dK, dV
template <typename T, int D, bool WIN = false, bool DROP = false>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(AttnBwdArgs<T> a) {
  const int win = WIN ? a.window : 0;  // sliding window (compiled out when WIN is false)
  constexpr int BQ = 64, BKV = 128;
  constexpr int LDT = BQ + pad_t<T>();
  constexpr int NC = D / 16, ND = D / 32;
  // Two LDS stages: the next query tile is stored while this one is consumed.
  __shared__ __attribute__((aligned(16))) T qs[2][BQ * Swz<T, D>::LD];
  __shared__ __attribute__((aligned(16))) T dos[2][BQ * Swz<T, D>::LD];
  __shared__ __attribute__((aligned(16))) T qts[2][D * LDT];
  __shared__ __attribute__((aligned(16))) T dots[2][D * LDT];
  __shared__ __attribute__((aligned(16))) float lse_s[2][BQ];
  __shared__ __attribute__((aligned(16))) float dd_s[2][BQ];

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
    kf[c] = kvrow < s ? ld_frag(Kp + (int64_t)kvrow * D + 16 * c + 8 * g) : zero_frag<T>();
    vf[c] = kvrow < s ? ld_frag(Vp + (int64_t)kvrow * D + 16 * c + 8 * g) : zero_frag<T>();
  }

  f32x16 dkacc[ND], dvacc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) { dkacc[i] = zero16(); dvacc[i] = zero16(); }

  const int nqt = (s + BQ - 1) / BQ;
  const int qt0 = a.causal ? kv0 / BQ : 0;
  // Sliding window: queries past kv0 + BKV - 1 + W - 1 see none of these keys.
  const int qt1 = win ? min(nqt, (kv0 + BKV + win - 2) / BQ + 1) : nqt;
  const int per_head = qt1 - qt0;
  const int nsteps = per_head * a.group;

  RowTile<T, BQ, D> qtile, dotile;
  float lse_r = 0.f, dd_r = 0.f;
  auto load_step = [&](int step) {
    const int hq = hk * a.group + step / per_head;
    const int q0 = (qt0 + step % per_head) * BQ;
    qtile.load(a.q + (int64_t)hq * s * D, D, q0, s, tid);
    dotile.load(a.dout + (int64_t)hq * D, a.lddo, q0, s, tid);
    if (tid < BQ) {
      const int qr = q0 + tid;
      lse_r = qr < s ? a.lse[(int64_t)hq * s + qr] : INFINITY;
      dd_r = qr < s ? a.dvec[(int64_t)hq * s + qr] : 0.f;
    }
  };
  auto store_step = [&](int buf) {
    qtile.store_swz(qs[buf], tid);
    qtile.store_cols(qts[buf], LDT, tid);
    dotile.store_swz(dos[buf], tid);
    dotile.store_cols(dots[buf], LDT, tid);
    if (tid < BQ) { lse_s[buf][tid] = lse_r; dd_s[buf][tid] = dd_r; }
  };
  if (nsteps > 0) {
    load_step(0);
    store_step(0);
  }
  __syncthreads();

  for (int step = 0; step < nsteps; ++step) {
    const int q0 = (qt0 + step % per_head) * BQ;
    const int buf = step & 1;
    if (step + 1 < nsteps) load_step(step + 1);
    const T* qsb = qs[buf];
    const T* dosb = dos[buf];
    const T* qtsb = qts[buf];
    const T* dotsb = dots[buf];
    const float* lseb = lse_s[buf];
    const float* ddb = dd_s[buf];

    // Steps touching the diagonal (or the sequence end) need the mask.
    const bool MASK = (a.causal && kv0 + BKV - 1 > q0) || kv0 + BKV - 1 >= s ||
                      (win && q0 + BQ - 1 >= kv0 + win);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // S = Q K^T and dP = dO V^T for this wave's 32 keys (lane = key).
      f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        sacc = mma(Swz<T, D>::frag(qsb, 32 * qb + lr, 16 * c + 8 * g), kf[c], sacc);
        dpacc = mma(Swz<T, D>::frag(dosb, 32 * qb + lr, 16 * c + 8 * g), vf[c], dpacc);
      }
      // Row terms of rows acc_row(4k..4k+3) are 4 consecutive floats.
      f32x4 l4[4], d4[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        l4[k] = ld<f32x4>(&lseb[32 * qb + 8 * k + 4 * g]);
        d4[k] = ld<f32x4>(&ddb[32 * qb + 8 * k + 4 * g]);
      }
      if constexpr (DROP) {
        // dV takes the kept probabilities (scaled at the end); dS = P (z dP~ - D)
        // with z = scale for kept and 0 for dropped elements.
        const int hg = a.drop.head0 + hk * a.group + step / per_head;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const Philox4 rw = philox4x32_10((uint32_t)((q0 + 32 * qb + 8 * j + 4 * g) >> 2),
                                           (uint32_t)(kvrow >> 2), (uint32_t)hg,
                                           (uint32_t)a.drop.batch, a.drop.seed_lo, a.drop.seed_hi);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * j + e;
            const bool keep = drop_keep_byte(rw.w[e], kvrow & 3, a.drop.thr);
            const float p = fast_exp2(sacc[r] - l4[j][e]);
            sacc[r] = keep ? p : 0.f;
            dpacc[r] = p * ((keep ? a.drop.scale : 0.f) * dpacc[r] - d4[j][e]);
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(sacc[r] - l4[r >> 2][r & 3]);
          sacc[r] = p;
          dpacc[r] = p * (dpacc[r] - d4[r >> 2][r & 3]);
        }
      }
      // Causal / tail / window mask: key row must be <= min(query, s - 1) and,
      // with a window, more than query - W.
      if (MASK && ((a.causal && kv0 + 32 * w + 31 > q0 + 32 * qb) || kv0 + 32 * w + 31 >= s ||
                   (win && q0 + 32 * qb + 31 >= kv0 + 32 * w + win))) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qg = q0 + 32 * qb + acc_row(r, g);
          const bool masked = kvrow > (a.causal ? min(qg, s - 1) : s - 1) ||
                              (win && kvrow <= qg - win);
          sacc[r] = masked ? 0.f : sacc[r];
          dpacc[r] = masked ? 0.f : dpacc[r];
        }
      }
      // dV += P^T dO and dK += dS^T Q, A operands straight from registers.
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int cc = 2 * qb + h2;
        float tp[8], td[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          tp[e] = sacc[8 * h2 + e];
          td[e] = dpacc[8 * h2 + e];
        }
        const auto pa = pack_frag<T>(tp);
        const auto dsa = pack_frag<T>(td);
#pragma unroll
        for (int i = 0; i < ND; ++i) {
          const T* dor = &dotsb[(32 * i + lr) * LDT + 16 * cc + 4 * g];
          dvacc[i] = mma(pa, ld_frag_split(dor, dor + 8), dvacc[i]);
          const T* qr = &qtsb[(32 * i + lr) * LDT + 16 * cc + 4 * g];
          dkacc[i] = mma(dsa, ld_frag_split(qr, qr + 8), dkacc[i]);
        }
      }
    }
    if (step + 1 < nsteps) store_step(buf ^ 1);
    __syncthreads();
  }

  // dK (scaled, inverse RoPE) and dV to the token-major outputs.
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    const int d = 32 * i + lr;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kv = kv0 + 32 * w + acc_row(r, g);
      float dkv = dkacc[i][r] * a.dk_scale;
      const float pair = shfl_xor(dkv, 1);
      if (a.rope && kv < s) {
        const float2 cs = a.rope[(int64_t)kv * (D / 2) + (d >> 1)];
        dkv = (d & 1) ? (dkv * cs.x - pair * cs.y) : (dkv * cs.x + pair * cs.y);
      }
      if (kv < s) {
        a.dk[(int64_t)kv * a.lddkv + (int64_t)hk * D + d] = from_f32<T>(dkv);
        a.dv[(int64_t)kv * a.lddkv + (int64_t)hk * D + d] =
            from_f32<T>(DROP ? dvacc[i][r] * a.drop.scale : dvacc[i][r]);
      }
    }
  }
}

// ============================================================================ backward: dQ
template <typename T, int D, bool WIN = false, bool DROP = false>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(AttnBwdArgs<T> a) {
  const int win = WIN ? a.window : 0;  // sliding window (compiled out when WIN is false)
  constexpr int BQ = 128, BKV = 64;
  constexpr int LDT = BKV + pad_t<T>();
  constexpr int NC = D / 16, ND = D / 32;
  __shared__ __attribute__((aligned(16))) T ks[BKV * Swz<T, D>::LD];
  __shared__ __attribute__((aligned(16))) T vs[BKV * Swz<T, D>::LD];
  __shared__ __attribute__((aligned(16))) T kts[D * LDT];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, g = lane >> 5;
  const int s = a.s;
  const int nqt = (s + BQ - 1) / BQ;
  int hq, qt;
  map_head_tile(blockIdx.x, a.nh, nqt, a.causal != 0, hq, qt);
  const int hk = hq / a.group;
  const int q0 = qt * BQ;
  const int qrow = q0 + 32 * w + lr;
  const T* Kp = a.k + (int64_t)hk * s * D;
  const T* Vp = a.v + (int64_t)hk * s * D;

  // This wave's 32 query rows of Q and dO as B operands (lane = query row).
  typename Frag<T>::type qf[NC], df[NC];
  const T* Qp = a.q + (int64_t)hq * s * D;
  const T* dOp = a.dout + (int64_t)hq * D;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    qf[c] = qrow < s ? ld_frag(Qp + (int64_t)qrow * D + 16 * c + 8 * g) : zero_frag<T>();
    df[c] = qrow < s ? ld_frag(dOp + (int64_t)qrow * a.lddo + 16 * c + 8 * g) : zero_frag<T>();
  }
  const float lse_q = qrow < s ? a.lse[(int64_t)hq * s + qrow] : INFINITY;
  const float dd_q = qrow < s ? a.dvec[(int64_t)hq * s + qrow] : 0.f;

  const int kv_end = a.causal ? min(s, q0 + BQ) : s;
  const int ntiles = (kv_end + BKV - 1) / BKV;
  const bool wave_active = q0 + 32 * w < s;
  const int wave_last = min(q0 + 32 * w + 31, s - 1);
  const int wave_tiles = a.causal ? wave_last / BKV + 1 : ntiles;
  const int t_lo = win ? max(0, q0 - win + 1) / BKV : 0;
  const int wave_t_lo = win ? max(0, q0 + 32 * w - win + 1) / BKV : 0;

  RowTile<T, BKV, D> ktile, vtile;
  f32x16 dqacc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) dqacc[i] = zero16();

  if (ntiles > t_lo) {
    ktile.load(Kp, D, t_lo * BKV, s, tid);
    vtile.load(Vp, D, t_lo * BKV, s, tid);
  }
  for (int t = t_lo; t < ntiles; ++t) {
    __syncthreads();
    ktile.store_swz(ks, tid);
    ktile.store_cols(kts, LDT, tid);
    vtile.store_swz(vs, tid);
    __syncthreads();
    if (t + 1 < ntiles) {
      ktile.load(Kp, D, (t + 1) * BKV, s, tid);
      vtile.load(Vp, D, (t + 1) * BKV, s, tid);
    }
    if (wave_active && t < wave_tiles && t >= wave_t_lo) {
      const int kvb = t * BKV;
      const bool MASK = (a.causal ? (kvb + BKV - 1 > q0 + 32 * w) : (kvb + BKV > s)) ||
                        (win && kvb <= q0 + 32 * w + 31 - win);
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        // S^T = K Q^T and dP^T = V dO^T (lane = query row).
        f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          sacc = mma(Swz<T, D>::frag(ks, 32 * sb + lr, 16 * c + 8 * g), qf[c], sacc);
          dpacc = mma(Swz<T, D>::frag(vs, 32 * sb + lr, 16 * c + 8 * g), df[c], dpacc);
        }
        if constexpr (DROP) {  // dS = P (z dP~ - D), z = scale (kept) or 0
          const int hg = a.drop.head0 + hq;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t wd = drop_word(a.drop, qrow >> 2, (kvb + 32 * sb + 8 * j + 4 * g) >> 2,
                                          hg, qrow & 3);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * j + e;
              const float p = fast_exp2(sacc[r] - lse_q);
              const float z = drop_keep_byte(wd, e, a.drop.thr) ? a.drop.scale : 0.f;
              dpacc[r] = p * (z * dpacc[r] - dd_q);
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(sacc[r] - lse_q);
            dpacc[r] = p * (dpacc[r] - dd_q);
          }
        }
        if (MASK) {  // wave-uniform; keys outside [query - W + 1, min(query, s - 1)] contribute nothing
          const int qc = a.causal ? min(qrow, s - 1) : s - 1;
          const int lim = qc - kvb - 32 * sb;
          const int lo = win ? qc - win - kvb - 32 * sb : -BKV;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            dpacc[r] = (acc_row(r, g) > lim || acc_row(r, g) <= lo) ? 0.f : dpacc[r];
        }
        // dQ^T += K^T dS^T over this block's 32 keys (two 16-key chunks).
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int cc = 2 * sb + h2;
          float td[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) td[e] = dpacc[8 * h2 + e];
          const auto dsf = pack_frag<T>(td);
#pragma unroll
          for (int i = 0; i < ND; ++i) {
            const T* row = &kts[(32 * i + lr) * LDT + 16 * cc + 4 * g];
            dqacc[i] = mma(ld_frag_split(row, row + 8), dsf, dqacc[i]);
          }
        }
      }
    }
  }

  // dQ = scale * dQ^T, inverse RoPE on (d, d^1) = registers (r, r^1).
  if (wave_active && qrow < s) {
    T* out = a.dq + (int64_t)qrow * a.lddq + (int64_t)hq * D;
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * i + r4 * 8 + 4 * g;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = dqacc[i][4 * r4 + e] * a.scale;
        if (a.rope) {
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            const float2 cs = a.rope[(int64_t)qrow * (D / 2) + ((d0 + e) >> 1)];
            const float ev = v[e], od = v[e + 1];
            v[e] = ev * cs.x + od * cs.y;
            v[e + 1] = -ev * cs.y + od * cs.x;
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) out[d0 + e] = from_f32<T>(v[e]);
      }
  }
}

}  // namespace bpt
