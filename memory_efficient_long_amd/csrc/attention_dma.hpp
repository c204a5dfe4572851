// bf16 attention kernels (head_dim 64 / 128) whose key/value and query tiles
// travel global -> LDS by direct LDS loads (global_load_lds_dwordx4: lane l's
// 16 bytes land at the instruction's LDS base + 16 l; see dma16_s), so no register staging
// and no in-register transposes are needed. Tiles are row-major, unpadded,
// with the 16-byte chunks of row r XOR-permuted by f(r) (see DmaTile) so
// that both read forms are free of bank conflicts on the 64-bank LDS: a
// 16-byte row-fragment read serves 16 lanes (16 consecutive rows, one chunk
// each) per cycle, a transpose read 32 lanes (4 consecutive rows, 64
// contiguous bytes each). Operands
// that need the transposed tile (V^T in the forward, dO^T and Q^T in the
// dK/dV pass, K^T in the dQ pass) are read with ds_read_b64_tr_b16, which,
// within each 16-lane group, gives lane i element (i % 4) of the 8-byte piece
// addressed by lane 4e + i / 4 as its element e: one read yields four
// consecutive rows of one column per lane.
//
// The computation is the one documented in attention.hpp (same tiling, same
// lane-local softmax statistics, same permuted reduction order); only the
// staging differs. Register use drops enough for two waves per SIMD in all
// three kernels.
#pragma once

#include "attention.hpp"

namespace bpt {

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D>
struct DmaTile {
  static constexpr int RB = D * 2;   // row bytes (bf16)
  static constexpr int CPR = D / 8;  // 16-byte chunks per row
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  // D = 128 (one row per 256-byte bank line): f = 4 (r & 3) + ((r >> 2) & 3)
  // is a bijection on 16 consecutive rows, and its high two bits separate
  // the 4-chunk groups of 4 consecutive rows. D = 64 (two rows per line):
  // f = 4 ((r >> 1) & 1) + ((r >> 2) & 3) does the same with the row parity
  // selecting the half line. Both satisfy f(r + 8) = f(r) ^ 2, so the
  // second half of a transpose fragment sits at the first address ^ 32.
  __device__ static __forceinline__ int f(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
  // Tile layout: row r (RB bytes) holds its 16-byte chunk c at byte
  // r RB + 16 (c ^ f(r)). Tiles are 1024-byte aligned.
  //
  // Fragment reads from a per-lane constant base: the chunk permutation is an
  // XOR on bits that lie below the row stride, so every fragment of a lane is
  // its base XOR a compile-time constant plus a constant offset (one base
  // register per read form instead of one address per fragment).
  //   row fragment (row 32 blk + lane % 32, elements 16 c + 8 g .. + 7):
  //     tile + 32 blk RB + (rf ^ 32 c)
  //   transposed-operand fragment for output column n = 32 i + lane % 32 and
  //   reduction chunk cc (elements 0-3 = rows 16 cc + 4 g + {0..3}, elements
  //   4-7 = rows 16 cc + 8 + 4 g + {0..3}, all at column n), two 8-byte
  //   transpose reads:
  //     a0 = tile + 16 cc RB + (tr ^ 64 i), a1 = (a0 ^ 32) + 8 RB
  //   (XOR-ing the byte address by 32 flips bit 1 of the chunk index, and
  //   f(r + 8) = f(r) ^ 2).
  __device__ static __forceinline__ uint32_t rf_base(int lane) {
    const int lr = lane & 31, g = lane >> 5, F = f(lr);
    return lr * RB + 32 * (F >> 1) + 16 * (g ^ (F & 1));
  }
  __device__ static __forceinline__ uint32_t tr_base(int lane) {
    const int li = lane & 15, g = lane >> 5, half = (lane >> 4) & 1;
    const int r = 4 * g + (li >> 2), F = f(r), x = 2 * half + ((li & 3) >> 1);
    return r * RB + 64 * (F >> 2) + 16 * (x ^ (F & 3)) + 8 * (li & 1);
  }
  __device__ static __forceinline__ bf16x8 frag_at(uint32_t tile, uint32_t rf, int blk, int c) {
    return *(const __attribute__((address_space(3))) bf16x8*)(size_t)(tile + 32 * blk * RB +
                                                                       (rf ^ (32u * c)));
  }
  // SPLIT: the second address as its own constant + (tr ^ (64 i + 32)) (tile
  // + 16 cc RB is a multiple of 256, so this equals the first address ^ 32,
  // plus 8 rows) -- one XOR per read with no dependence on the first address;
  // otherwise derived from the first address.
  template <bool SPLIT = true>
  __device__ static __forceinline__ bf16x8 tr_at(uint32_t tile, uint32_t tr, int cc, int i) {
    const uint32_t a0 = tile + 16 * cc * RB + (tr ^ (64u * i));
    const uint32_t a1 = SPLIT ? tile + 16 * cc * RB + 8 * RB + (tr ^ (64u * i + 32u))
                              : (a0 ^ 32u) + 8 * RB;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(size_t)a0);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(size_t)a1);
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
  }

  // ---- Direct loads of R-row tiles (NW waves) with a per-lane constant
  // offset: load m of wave w covers rows brow = (w PERW + m) RPI + lane / CPR,
  // and f(brow + j) = f(brow) ^ f(j) for j < RPI, so the global chunk is
  // (lane % CPR) ^ f(lane / CPR) ^ f(brow) with the last term wave-uniform.
  // Requires the row stride (in bytes) to be a multiple of RB.
  template <int R, int NW>
  struct Loader {
    static constexpr int PERW = R * RB / 1024 / NW, RPI = 1024 / RB;
    static_assert(PERW >= 1 && R * RB % (1024 * NW) == 0, "tile split");
    uint32_t l0;
    int64_t ldb;
    __device__ __forceinline__ Loader(int64_t ld, int lane) : ldb(ld * 2) {
      const int j = lane / CPR;
      l0 = (uint32_t)(j * ldb) + 16u * ((lane % CPR) ^ f(j));
    }
    // Rows [row0, row0 + R) of src into the tile at LDS address `tile`; rows
    // at or past rlim repeat row rlim - 1 (masked by the caller). LAZY: the
    // lane offset is recomputed from the lane id here instead of being read
    // from l0, for kernels where keeping it live across the loop would spill
    // it (a spill reload after these loads would wait for them).
    template <bool LAZY = false>
    __device__ __forceinline__ void issue(uint32_t tile, const bf16* src, int row0, int rlim, int w,
                                          int lane) const {
      // The empty asm statements make the lane values opaque at each call, so
      // the per-load offsets are recomputed here (one VALU op each) rather
      // than hoisted out of the caller's loop into registers of their own.
      if (row0 + R <= rlim) {
        uint32_t l;
        if constexpr (LAZY) {
          int ln = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
          asm volatile("" : "+v"(ln));
          const int j = ln / CPR;
          l = (uint32_t)(j * ldb) + 16u * ((ln % CPR) ^ f(j));
        } else {
          l = l0;
        }
        asm volatile("" : "+v"(l));
        const char* base = (const char*)src + (int64_t)row0 * ldb;
#pragma unroll
        for (int m = 0; m < PERW; ++m) {
          const int brow = (w * PERW + m) * RPI;
          dma16_s(base + brow * ldb, l ^ (16u * f(brow)), tile + (w * PERW + m) * 1024);
        }
      } else {
        int ln = LAZY ? (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u))
                      : lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int m = 0; m < PERW; ++m) {
          const int o = (w * PERW + m) * 1024 + 16 * ln;
          const int r = o / RB, p = (o % RB) >> 4;
          const int gr = min(row0 + r, rlim - 1);
          dma16_v((const char*)src + gr * ldb + ((p ^ f(r)) << 4), tile + (w * PERW + m) * 1024);
        }
      }
    }
  };
};


__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0); }

// ============================================================================ forward
template <int D, bool WIN = false, bool DROP = false>
__global__ __launch_bounds__(256, 2) void attn_fwd_dma_kernel(AttnFwdArgs<bf16> a) {
  const int win = WIN ? a.window : 0;  // sliding window (compiled out when WIN is false)
  using TL = DmaTile<D>;
  constexpr int BQ = 128, BKV = 64;
  constexpr int NC = D / 16, ND = D / 32;
  __shared__ __attribute__((aligned(1024))) bf16 ks[2][BKV * D];
  __shared__ __attribute__((aligned(1024))) bf16 vs[2][BKV * D];
  constexpr uint32_t TB = BKV * D * 2;  // tile bytes

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, g = lane >> 5;
  const int s = a.s;
  const int nqt = (s + BQ - 1) / BQ;
  int hq, qt;
  map_head_tile(blockIdx.x, a.nh, nqt, a.causal != 0, hq, qt);
  const int hk = hq / a.group;
  const int q0 = qt * BQ;
  const int qrow = q0 + 32 * w + lr;
  const bf16* Qp = a.q + (int64_t)hq * s * D;
  const bf16* Kp = a.k + (int64_t)hk * s * D;
  const bf16* Vp = a.v + (int64_t)hk * s * D;

  bf16x8 qf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
    qf[c] = qrow < s ? ld_frag(Qp + (int64_t)qrow * D + 16 * c + 8 * g) : zero_frag<bf16>();

  const int kv_end = a.causal ? min(s, q0 + BQ) : s;
  const int ntiles = (kv_end + BKV - 1) / BKV;
  const bool wave_active = q0 + 32 * w < s;
  const int wave_last = min(q0 + 32 * w + 31, s - 1);
  const int wave_tiles = a.causal ? wave_last / BKV + 1 : ntiles;
  // Sliding window: key tiles wholly before every row's window are skipped
  // (the workgroup's first row bounds t_lo, each wave's its own).
  const int t_lo = win ? max(0, q0 - win + 1) / BKV : 0;
  const int wave_t_lo = win ? max(0, q0 + 32 * w - win + 1) / BKV : 0;

  f32x16 oacc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) oacc[i] = zero16();
  // Q carries log2(e)/sqrt(D): the products are base-2 scores, and P is
  // exp2(S - m) with no per-element scaling. (Seeding the S accumulators
  // with -m, which would save the subtraction too, costs 16 registers that
  // this kernel does not have: it measured slower.)
  float m_run = -INFINITY, l_run = 0.f;

  const uint32_t ksa = lds_addr(&ks[0][0]), vsa = lds_addr(&vs[0][0]);
  const uint32_t rf = TL::rf_base(lane), trb = TL::tr_base(lane);
  const typename TL::template Loader<BKV, 4> kvld(D, lane);
  if (ntiles > t_lo) {
    kvld.issue(ksa, Kp, t_lo * BKV, s, w, lane);
    kvld.issue(vsa, Vp, t_lo * BKV, s, w, lane);
  }
  wait_dma();
  __syncthreads();

  // One key tile per call; the buffer index is a compile-time constant (the
  // loop below is unrolled by two), so every LDS address is a per-lane base
  // held in a register plus an immediate offset.
  auto tile_step = [&](int t, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    if (t + 1 < ntiles) {
      kvld.issue(ksa + (buf ^ 1) * TB, Kp, (t + 1) * BKV, s, w, lane);
      kvld.issue(vsa + (buf ^ 1) * TB, Vp, (t + 1) * BKV, s, w, lane);
    }
    if (wave_active && t < wave_tiles && t >= wave_t_lo) {
      const int kvb = t * BKV;
      const bool MASK = (a.causal ? (kvb + BKV - 1 > q0 + 32 * w) : (kvb + BKV > s)) ||
                        (win && kvb <= q0 + 32 * w + 31 - win);
      f32x16 sacc[2] = {zero16(), zero16()};
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
          sacc[sb] = mma(TL::frag_at(ksa + buf * TB, rf, sb, c), qf[c], sacc[sb]);
      // Order hint (sched_group_barrier; 0x100 = LDS reads, 0x008 = MFMA):
      // each K fragment is read two MFMAs before its use instead of right
      // before it.
      {
        constexpr int PF = 2;
        __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
        for (int m = 0; m < 2 * NC - PF; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
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
      // A query's 64 keys of the tile are split between lanes l and l + 32;
      // each half tests its own maximum (the running max is common to both),
      // and the two are combined (an LDS shuffle) only on the rare tiles
      // where the running max must move.
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[sb][r]);
      if (__any(mx > m_run + 8.f)) {  // move the running max only by > 2^8
        const float m_new = fmaxf(m_run, fmaxf(mx, shfl_xor(mx, 32)));
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
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[sb][r] = fast_exp2(sacc[sb][r] - m_sub);
      // P in bf16 (the B operand of O^T += V^T P^T); the row sum is taken
      // over the same bf16 values, two per dot-product instruction, so the
      // normaliser matches what the MFMAs accumulate.
      bf16x8 pf[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        float tmp[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) tmp[e] = sacc[cc >> 1][8 * (cc & 1) + e];
        pf[cc] = pack_frag<bf16>(tmp);
      }
      // this half's 32 keys; the halves share the running max and are added
      // once, after the last tile
      l_run += row_sum_bf16x32(pf);
      if constexpr (DROP) {
        // The normaliser above is the undropped one; dropped probabilities are
        // cleared in the packed fragments (element e of pf[cc] is key
        // 32 (cc / 2) + 8 (2 (cc % 2) + e / 4) + 4 g + e % 4 of the tile) and
        // the kept ones scaled once, in the output.
        // Key group (4 keys) kvb / 4 + 2 m + g for m = 2 cc + half; the calls
        // for m = 4 rd + j are shared by the quad (lane j computes it).
        const int hg = a.drop.head0 + hq;
        uint32_t wds[2][4];
#pragma unroll
        for (int rd = 0; rd < 2; ++rd)
          drop_words_rows(a.drop, qrow >> 2, (kvb >> 2) + 2 * (4 * rd + (lane & 3)) + g, hg, lane,
                          wds[rd]);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          u32x4 wv = __builtin_bit_cast(u32x4, pf[cc]);
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int m = 2 * cc + half;
            const uint32_t wd = wds[m >> 2][m & 3];
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
              const uint32_t lo = drop_keep_byte(wd, 2 * pr, a.drop.thr) ? 0x0000FFFFu : 0u;
              const uint32_t hi = drop_keep_byte(wd, 2 * pr + 1, a.drop.thr) ? 0xFFFF0000u : 0u;
              wv[2 * half + pr] &= lo | hi;
            }
          }
          pf[cc] = __builtin_bit_cast(bf16x8, wv);
        }
      }
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
#pragma unroll
        for (int i = 0; i < ND; ++i)
          oacc[i] = mma(TL::template tr_at<false>(vsa + buf * TB, trb, cc, i), pf[cc], oacc[i]);
      // The V^T pair of each product one MFMA ahead (two measured slower).
      {
        constexpr int PF = 1;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
        for (int m = 0; m < 4 * ND - PF; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
      }
    }
    wait_dma();
    __syncthreads();
  };
  for (int t = t_lo; t < ntiles; t += 2) {
    tile_step(t, std::integral_constant<int, 0>());
    if (t + 1 < ntiles) tile_step(t + 1, std::integral_constant<int, 1>());
  }

  l_run += shfl_xor(l_run, 32);  // both halves' sums
  if (wave_active && qrow < s) {
    const float inv_l = (DROP ? a.drop.scale : 1.f) / l_run;
    bf16* orow = a.o + (int64_t)qrow * a.ldo + (int64_t)hq * D;
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * i + r4 * 8 + 4 * g;
#pragma unroll
        for (int e = 0; e < 4; ++e) orow[d + e] = (bf16)(oacc[i][4 * r4 + e] * inv_l);
      }
    if (g == 0) a.lse[(int64_t)hq * s + qrow] = m_run + __log2f(l_run);
  }
}

// Value of lane R of this lane's 16-lane row (DPP row_newbcast). Every source
// lane is valid, so the move keeps no old value: without bound_ctrl the
// compiler first initialises each destination with a separate move.
template <int R>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + R, 0xF, 0xF, true));
}
template <int... R>
__device__ __forceinline__ void seed_rows(f32x16& s, f32x16& d, float xs, float xd,
                                          std::integer_sequence<int, R...>) {
  ((s[R] = row_bcast<R>(xs), d[R] = row_bcast<R>(xd)), ...);
}

// Dropout in the dK/dV pass for one 32-query block: element r = 4 j + e of
// the lane's accumulators is query 4 (q4 + 2 j) + e (q4 = (q0 + 32 qb + 4 g) / 4)
// and key kvrow; -D of that query is broadcast from lane r of the 16-lane row
// (xd holds -D of query n16 of the row, as for the seeds).
template <int... J>
__device__ __forceinline__ void drop_dkdv(f32x16& sacc, f32x16& dpacc, float xd, const DropArgs& d,
                                          int q4, int kvrow, int hg,
                                          std::integer_sequence<int, J...>) {
  // the four query groups' calls are shared by the quad (lane i computes
  // group q4 + 2 i); bq[j] holds this key's byte of each word of group j
  uint32_t bq[4];
  drop_bytes_cols(d, q4 + 2 * (kvrow & 3), kvrow >> 2, hg, kvrow, bq);  // kvrow % 4 = lane % 4
  auto group = [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    auto elem = [&](auto ec) {
      constexpr int e = decltype(ec)::value, r = 4 * j + e;
      const bool keep = drop_keep_byte(bq[j], e, d.thr);
      const float p = fast_exp2(sacc[r]);
      sacc[r] = keep ? p : 0.f;
      dpacc[r] = p * fmaf(keep ? d.scale : 0.f, dpacc[r], row_bcast<r>(xd));
    };
    elem(std::integral_constant<int, 0>());
    elem(std::integral_constant<int, 1>());
    elem(std::integral_constant<int, 2>());
    elem(std::integral_constant<int, 3>());
  };
  (group(std::integral_constant<int, J>()), ...);
}

// ============================================================================ backward: dK, dV
// SPLIT: the query-head-split variant (a.nparts > 1, partial sums to a.part);
// without it the part index is a compile-time zero and nothing of the split
// remains in the code.
template <int D, bool SPLIT = false, bool WIN = false, bool DROP = false>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkdv_dma_kernel(AttnBwdArgs<bf16> a) {
  const int win = WIN ? a.window : 0;  // sliding window (compiled out when WIN is false)
  using TL = DmaTile<D>;
  constexpr int BQ = 64, BKV = 128;
  constexpr int NC = D / 16, ND = D / 32;
  __shared__ __attribute__((aligned(1024))) bf16 qs[2][BQ * D];
  __shared__ __attribute__((aligned(1024))) bf16 dos[2][BQ * D];
  __shared__ __attribute__((aligned(16))) float lse_s[2][BQ];
  constexpr uint32_t TB = BQ * D * 2;  // tile bytes
  __shared__ __attribute__((aligned(16))) float dd_s[2][BQ];

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, g = lane >> 5;
  const int s = a.s;
  const int nkt = (s + BKV - 1) / BKV;
  // Workgroup (KV head, part, key tile): part pp covers query heads
  // [pp gp, (pp + 1) gp) of the KV head's group, gp = group / nparts.
  const int np = SPLIT ? a.nparts : 1, gp = SPLIT ? a.group / np : a.group;
  int vh, kt;
  map_head_tile(blockIdx.x, a.nkv * np, nkt, false, vh, kt);
  const int hk = SPLIT ? vh / np : vh, pp = SPLIT ? vh - hk * np : 0;
  const int kv0 = kt * BKV;
  const int kvrow = kv0 + 32 * w + lr;
  const bf16* Kp = a.k + (int64_t)hk * s * D;
  const bf16* Vp = a.v + (int64_t)hk * s * D;

  bf16x8 kf[NC], vf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    kf[c] = kvrow < s ? ld_frag(Kp + (int64_t)kvrow * D + 16 * c + 8 * g) : zero_frag<bf16>();
    vf[c] = kvrow < s ? ld_frag(Vp + (int64_t)kvrow * D + 16 * c + 8 * g) : zero_frag<bf16>();
  }
  // The last KPARK K fragments are parked in LDS and read back where they are
  // used: the registers they free keep the loop free of spills (whose reloads,
  // counted with the direct loads by vmcnt, would wait for the tile loads) and
  // leave room to read fragments ahead of their MFMAs. Three measured best
  // (12 KiB per workgroup; four would leave room for only one workgroup per CU).
  constexpr int KPARK = 3;
  __shared__ __attribute__((aligned(16))) bf16x8 kpark[KPARK > 0 ? KPARK : 1][4][64];
#pragma unroll
  for (int c = 0; c < KPARK; ++c) kpark[c][w][lane] = kf[NC - KPARK + c];
  const uint32_t kpa = lds_addr(&kpark[0][w][lane]);

  f32x16 dkacc[ND], dvacc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) { dkacc[i] = zero16(); dvacc[i] = zero16(); }

  const int nqt = (s + BQ - 1) / BQ;
  const int qt0 = a.causal ? kv0 / BQ : 0;
  // Sliding window: queries past kv0 + BKV - 1 + W - 1 see none of these keys.
  const int qt1 = win ? min(nqt, (kv0 + BKV + win - 2) / BQ + 1) : nqt;
  const int per_head = qt1 - qt0;
  const int nsteps = per_head * gp;
  // Query tiles are visited from the last one down: the workgroups resident
  // on an XCD (consecutive key tiles of one head) then start on the same tile
  // and sweep the head's Q and dO together through that XCD's L2, instead of
  // starting two tiles apart each (a spread that outgrows the L2 along the way).
  auto q_tile = [&](int step) { return qt1 - 1 - step % per_head; };

  // Row statistics of the next step: loaded raw (before the tile loads, so
  // waiting for them never waits for the tiles) and converted when stored.
  float lse_r = 0.f, dd_r = 0.f;
  bool valid_r = false;
  const uint32_t qsa = lds_addr(&qs[0][0]), dosa = lds_addr(&dos[0][0]);
  uint32_t rf = TL::rf_base(lane), trb = TL::tr_base(lane);
  const typename TL::template Loader<BQ, 4> qld(D, lane), dold(a.lddo, lane);
  auto load_step = [&](int step, int buf) {
    const int hq = hk * a.group + pp * gp + step / per_head;
    const int q0 = q_tile(step) * BQ;
    if (tid < BQ) {
      const int qr = q0 + tid;
      valid_r = qr < s;
      lse_r = valid_r ? a.lse[(int64_t)hq * s + qr] : 0.f;
      dd_r = valid_r ? a.dvec[(int64_t)hq * s + qr] : 0.f;
    }
    qld.template issue<true>(qsa + buf * TB, a.q + (int64_t)hq * s * D, q0, s, w, lane);
    dold.template issue<true>(dosa + buf * TB, a.dout + (int64_t)hq * D, q0, s, w, lane);
  };
  // Stored negated to seed the S and dP accumulators (S = Q K^T is in the
  // base-2 units of the LSE); rows past the end get -inf (P = 0) and 0.
  auto store_stats = [&](int buf) {
    if (tid < BQ) {
      lse_s[buf][tid] = valid_r ? -lse_r : -INFINITY;
      dd_s[buf][tid] = valid_r ? -dd_r : 0.f;
    }
  };
  if (nsteps > 0) {
    load_step(0, 0);
    store_stats(0);
  }
  wait_dma();
  __syncthreads();

  // One query tile per call with a compile-time buffer index (the loop is
  // unrolled by two): every LDS address is a constant plus a per-lane base
  // XOR an immediate. The bases are made opaque per step so that the XORs
  // stay next to their reads instead of occupying a register each.
  auto q_step = [&](int step, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int q0 = q_tile(step) * BQ;
    asm volatile("" : "+v"(rf), "+v"(trb));
    if (step + 1 < nsteps) load_step(step + 1, buf ^ 1);
    const bool MASK = (a.causal && kv0 + BKV - 1 > q0) || kv0 + BKV - 1 >= s ||
                      (win && q0 + BQ - 1 >= kv0 + win);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // Seeding the accumulators with -lse and -D_i puts the row
      // statistics where the products land, with no extra registers.
      f32x16 sacc, dpacc;
      float xd;
      {
        // Element r of a lane's accumulators is query 32 qb + 8 (r / 4) +
        // 4 g + r % 4: lane n of each 16-lane row reads the statistics of
        // query 32 qb + 8 (n / 4) + 4 g + n % 4 (one LDS read each), and
        // element r is broadcast from lane r of the row (g is constant
        // within a row) -- two 4-byte reads per query block instead of
        // eight 16-byte ones.
        const int n16 = lane & 15;
        const int qi = 32 * qb + (n16 >> 2) * 8 + 4 * g + (n16 & 3);
        const float xl = lse_s[buf][qi];
        xd = dd_s[buf][qi];
        // with dropout the dP accumulators start at 0 and -D is added per
        // element after the mask (dS = P (z dP~ - D))
        seed_rows(sacc, dpacc, xl, DROP ? 0.f : xd, std::make_integer_sequence<int, 16>());
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        bf16x8 kc = kf[c];
        if (c >= NC - KPARK) {
          uint32_t pa = kpa + (c - (NC - KPARK)) * (4 * 64 * 16);
          asm volatile("" : "+v"(pa));
          kc = *(const __attribute__((address_space(3))) bf16x8*)(size_t)pa;
        }
        sacc = mma(TL::frag_at(qsa + buf * TB, rf, qb, c), kc, sacc);
        dpacc = mma(TL::frag_at(dosa + buf * TB, rf, qb, c), vf[c], dpacc);
      }
      // Order hint (sched_group_barrier; 0x100 = LDS reads, 0x008 = MFMA): the
      // two statistics reads and the first PF fragment reads, then each MFMA
      // followed by the next fragment read, so a read is issued PF MFMAs before
      // its use instead of right before it (3 measured best of 2-4; 2 in the
      // split window variant, where a third read in flight spills).
      {
        constexpr int PF = SPLIT && WIN ? 2 : 3;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 + PF, 0);
#pragma unroll
        for (int m = 0; m < 2 * NC - PF; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
      }
      if constexpr (DROP) {
        // dV takes the kept probabilities (scaled at the end); dS = P (z dP~ - D)
        // with z = scale (kept) or 0. Element r is query q0 + 32 qb +
        // 8 (r / 4) + 4 g + r % 4: one generator call per four queries.
        const int hg = a.drop.head0 + hk * a.group + pp * gp + step / per_head;
        drop_dkdv(sacc, dpacc, xd, a.drop, (q0 + 32 * qb + 4 * g) >> 2, kvrow, hg,
                  std::make_integer_sequence<int, 4>());
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(sacc[r]);
          sacc[r] = p;
          dpacc[r] = p * dpacc[r];
        }
      }
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
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int cc = 2 * qb + h2;
        float tp[8], td[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          tp[e] = sacc[8 * h2 + e];
          td[e] = dpacc[8 * h2 + e];
        }
        const bf16x8 pa = pack_frag<bf16>(tp);
        const bf16x8 dsa = pack_frag<bf16>(td);
#pragma unroll
        for (int i = 0; i < ND; ++i) {
          dvacc[i] = mma(pa, TL::tr_at(dosa + buf * TB, trb, cc, i), dvacc[i]);
          dkacc[i] = mma(dsa, TL::tr_at(qsa + buf * TB, trb, cc, i), dkacc[i]);
        }
      }
      // Same for dV and dK: two transpose reads per MFMA.
      {
        constexpr int PF = 2;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
        for (int m = 0; m < 4 * ND - PF; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
      }
    }
    if (step + 1 < nsteps) store_stats(buf ^ 1);
    wait_dma();
    __syncthreads();
  };
  for (int step = 0; step < nsteps; step += 2) {
    q_step(step, std::integral_constant<int, 0>());
    if (step + 1 < nsteps) q_step(step + 1, std::integral_constant<int, 1>());
  }

  if constexpr (SPLIT) {  // raw partial sums; dkdv_reduce_kernel scales, rotates and converts
    float* pk = a.part + ((int64_t)(2 * pp) * a.nkv + hk) * s * D;
    float* pv = pk + (int64_t)a.nkv * s * D;
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      const int d = 32 * i + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kv = kv0 + 32 * w + acc_row(r, g);
        if (kv < s) {
          pk[(int64_t)kv * D + d] = dkacc[i][r];
          pv[(int64_t)kv * D + d] = DROP ? dvacc[i][r] * a.drop.scale : dvacc[i][r];
        }
      }
    }
    return;
  }
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
        a.dk[(int64_t)kv * a.lddkv + (int64_t)hk * D + d] = (bf16)dkv;
        a.dv[(int64_t)kv * a.lddkv + (int64_t)hk * D + d] =
            (bf16)(DROP ? dvacc[i][r] * a.drop.scale : dvacc[i][r]);
      }
    }
  }
}

// dK, dV of the query-head-split pass: sums the nparts raw partials in
// order, then applies the dK factor and the inverse RoPE to dK as the unsplit
// kernel does, and stores both in bf16. One thread per (row, KV head, pair of
// columns).
template <int D>
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(AttnBwdArgs<bf16> a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int s = a.s;
  if (t >= (int64_t)s * a.nkv * (D / 2)) return;
  const int dp = (int)(t % (D / 2));
  const int64_t rh = t / (D / 2);
  const int hk = (int)(rh % a.nkv), kv = (int)(rh / a.nkv);
  const int64_t slab = (int64_t)a.nkv * s * D;
  const int64_t off = ((int64_t)hk * s + kv) * D + 2 * dp;
  float k0 = 0.f, k1 = 0.f, v0 = 0.f, v1 = 0.f;
  for (int p = 0; p < a.nparts; ++p) {
    const float2 pk = *(const float2*)(a.part + 2 * p * slab + off);
    const float2 pv = *(const float2*)(a.part + (2 * p + 1) * slab + off);
    k0 += pk.x; k1 += pk.y; v0 += pv.x; v1 += pv.y;
  }
  k0 *= a.dk_scale; k1 *= a.dk_scale;
  if (a.rope) {
    const float2 cs = a.rope[(int64_t)kv * (D / 2) + dp];
    const float r0 = k0 * cs.x + k1 * cs.y, r1 = k1 * cs.x - k0 * cs.y;
    k0 = r0; k1 = r1;
  }
  bf16* dk = a.dk + (int64_t)kv * a.lddkv + (int64_t)hk * D + 2 * dp;
  bf16* dv = a.dv + (int64_t)kv * a.lddkv + (int64_t)hk * D + 2 * dp;
  dk[0] = (bf16)k0; dk[1] = (bf16)k1;
  dv[0] = (bf16)v0; dv[1] = (bf16)v1;
}

// ============================================================================ backward: dQ
template <int D, bool WIN = false, bool DROP = false>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_dma_kernel(AttnBwdArgs<bf16> a) {
  const int win = WIN ? a.window : 0;  // sliding window (compiled out when WIN is false)
  using TL = DmaTile<D>;
  constexpr int BQ = 128, BKV = 64;
  constexpr int NC = D / 16, ND = D / 32;
  __shared__ __attribute__((aligned(1024))) bf16 ks[2][BKV * D];
  __shared__ __attribute__((aligned(1024))) bf16 vs[2][BKV * D];
  constexpr uint32_t TB = BKV * D * 2;  // tile bytes

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, g = lane >> 5;
  const int s = a.s;
  const int nqt = (s + BQ - 1) / BQ;
  int hq, qt;
  map_head_tile(blockIdx.x, a.nh, nqt, a.causal != 0, hq, qt);
  const int hk = hq / a.group;
  const int q0 = qt * BQ;
  const int qrow = q0 + 32 * w + lr;
  const bf16* Kp = a.k + (int64_t)hk * s * D;
  const bf16* Vp = a.v + (int64_t)hk * s * D;

  bf16x8 qf[NC], df[NC];
  const bf16* Qp = a.q + (int64_t)hq * s * D;
  const bf16* dOp = a.dout + (int64_t)hq * D;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    qf[c] = qrow < s ? ld_frag(Qp + (int64_t)qrow * D + 16 * c + 8 * g) : zero_frag<bf16>();
    df[c] = qrow < s ? ld_frag(dOp + (int64_t)qrow * a.lddo + 16 * c + 8 * g) : zero_frag<bf16>();
  }
  const float lse_q = qrow < s ? a.lse[(int64_t)hq * s + qrow] : INFINITY;
  const float dd_q = qrow < s ? a.dvec[(int64_t)hq * s + qrow] : 0.f;
  // S^T accumulates onto -lse (Q carries log2(e)/sqrt(D), so the products
  // are base-2 scores and P = exp2(acc)); dP^T onto -D_i (this lane's
  // query), so dS = P * acc. With dropout, dS = P (z dP~ - D), z = scale
  // (kept) or 0, and dP^T starts at 0. Rows past the end: P = 0.
  f32x16 sseed, dseed;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    sseed[r] = -lse_q;
    dseed[r] = DROP ? 0.f : -dd_q;
  }

  const int kv_end = a.causal ? min(s, q0 + BQ) : s;
  const int ntiles = (kv_end + BKV - 1) / BKV;
  const bool wave_active = q0 + 32 * w < s;
  const int wave_last = min(q0 + 32 * w + 31, s - 1);
  const int wave_tiles = a.causal ? wave_last / BKV + 1 : ntiles;
  const int t_lo = win ? max(0, q0 - win + 1) / BKV : 0;
  const int wave_t_lo = win ? max(0, q0 + 32 * w - win + 1) / BKV : 0;

  f32x16 dqacc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) dqacc[i] = zero16();

  const uint32_t ksa = lds_addr(&ks[0][0]), vsa = lds_addr(&vs[0][0]);
  uint32_t rf = TL::rf_base(lane), trb = TL::tr_base(lane);
  const typename TL::template Loader<BKV, 4> kvld(D, lane);
  if (ntiles > t_lo) {
    kvld.issue(ksa, Kp, t_lo * BKV, s, w, lane);
    kvld.issue(vsa, Vp, t_lo * BKV, s, w, lane);
  }
  wait_dma();
  __syncthreads();

  // One key tile per call with a compile-time buffer index (unrolled by two):
  // LDS addresses are constants plus a per-lane base XOR an immediate; the
  // bases are opaque per tile so the XORs stay next to their reads rather
  // than taking a register each.
  auto tile_step = [&](int t, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    asm volatile("" : "+v"(rf), "+v"(trb));
    if (t + 1 < ntiles) {
      kvld.issue(ksa + (buf ^ 1) * TB, Kp, (t + 1) * BKV, s, w, lane);
      kvld.issue(vsa + (buf ^ 1) * TB, Vp, (t + 1) * BKV, s, w, lane);
    }
    if (wave_active && t < wave_tiles && t >= wave_t_lo) {
      const int kvb = t * BKV;
      const bool MASK = (a.causal ? (kvb + BKV - 1 > q0 + 32 * w) : (kvb + BKV > s)) ||
                        (win && kvb <= q0 + 32 * w + 31 - win);
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        f32x16 sacc = sseed, dpacc = dseed;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          sacc = mma(TL::frag_at(ksa + buf * TB, rf, sb, c), qf[c], sacc);
          dpacc = mma(TL::frag_at(vsa + buf * TB, rf, sb, c), df[c], dpacc);
        }
        // Order hints as in the dK/dV pass: K and V fragments read three
        // MFMAs ahead here, the K^T pairs of the dQ products below two (not
        // with dropout, whose extra registers they would spill).
        if constexpr (!DROP) {
          constexpr int PF = 3;
          __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
          for (int m = 0; m < 2 * NC - PF; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
        }
        if constexpr (DROP) {
          const int hg = a.drop.head0 + hq;
          // key group (kvb + 32 sb + 8 j + 4 g) / 4, shared by the quad
          uint32_t wds[4];
          drop_words_rows(a.drop, qrow >> 2, ((kvb + 32 * sb + 4 * g) >> 2) + 2 * (lane & 3), hg,
                          lane, wds);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t wd = wds[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * j + e;
              const float z = drop_keep_byte(wd, e, a.drop.thr) ? a.drop.scale : 0.f;
              dpacc[r] = fast_exp2(sacc[r]) * (z * dpacc[r] - dd_q);
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) dpacc[r] *= fast_exp2(sacc[r]);
        }
        if (MASK) {
          const int qc = a.causal ? min(qrow, s - 1) : s - 1;
          const int lim = qc - kvb - 32 * sb;
          const int lo = win ? qc - win - kvb - 32 * sb : -BKV;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            dpacc[r] = (acc_row(r, g) > lim || acc_row(r, g) <= lo) ? 0.f : dpacc[r];
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int cc = 2 * sb + h2;
          float td[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) td[e] = dpacc[8 * h2 + e];
          const bf16x8 dsf = pack_frag<bf16>(td);
#pragma unroll
          for (int i = 0; i < ND; ++i) dqacc[i] = mma(TL::tr_at(ksa + buf * TB, trb, cc, i), dsf, dqacc[i]);
        }
        if constexpr (!DROP) {
          constexpr int PF = 2;
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
          for (int m = 0; m < 2 * ND - PF; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
        }
      }
    }
    wait_dma();
    __syncthreads();
  };
  for (int t = t_lo; t < ntiles; t += 2) {
    tile_step(t, std::integral_constant<int, 0>());
    if (t + 1 < ntiles) tile_step(t + 1, std::integral_constant<int, 1>());
  }

  if (wave_active && qrow < s) {
    bf16* out = a.dq + (int64_t)qrow * a.lddq + (int64_t)hq * D;
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
        for (int e = 0; e < 4; ++e) out[d0 + e] = (bf16)v[e];
      }
  }
}

}  // namespace bpt
