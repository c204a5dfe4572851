// bf16 MFMA GEMM fed by direct global -> LDS loads, same contract and
// epilogues as gemm_kernel in gemm.hpp (C[m, n] = sum_k A(m, k) B(n, k)).
//
// Each operand tile is stored in LDS in its global orientation, unpadded:
//   K-major operand (A(m, k) = A[m * lda + k]): BMN rows of BK k values;
//     fragments (one row, 8 consecutive k) are single 16-byte LDS reads.
//   MN-major operand (A(m, k) = A[k * lda + m]): BK rows of BMN values;
//     fragments come from two ds_read_b64_tr_b16, each giving a lane four
//     consecutive k of its column.
// Both forms hand lane (r = lane % 32, g = lane / 32) the reduction indices
// 16 kk + 8 g + {0..7}, so any pair of layouts feeds the same MFMA.
//
// global_load_lds moves 16 bytes per lane into LDS at the instruction's base
// + 16 * lane, so the bank swizzle (16-byte chunks XOR-permuted per row) is
// applied by choosing which global chunk each lane fetches. Nothing is staged
// in registers, which lets the pipeline run STAGES deep: the loads of step
// kt + STAGES - 1 are in flight while step kt computes.
//
// Requirements (checked by the host): K % BK == 0, rows of K-major operands
// and the contiguous extent of MN-major operands multiple of 8 elements,
// 16-byte aligned base pointers and leading dimensions. M and N tails are
// handled by clamping the fetched rows / columns (the extra outputs are not
// stored).
#pragma once

#include "gemm.hpp"

namespace bpt {

namespace gdma {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Wait until at most N vector-memory operations of this wave are in flight
// (expcnt and lgkmcnt fields left at their maxima, i.e. not waited on).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// K-major tile: R rows x BK bf16.
template <int R, int BK>
struct KTile {
  static constexpr int RB = BK * 2;
  static constexpr int CPR = BK / 8;
  static constexpr int BYTES = R * RB;
  static constexpr int RPL = 16 / CPR;  // rows per 256-byte bank line
  // A 16-byte fragment read serves 16 lanes (16 consecutive rows) per cycle:
  // f is a bijection on the bank-line index of 16 consecutive rows.
  __device__ static __forceinline__ int f(int r) { return (r / RPL) & (CPR - 1); }

  // Per-lane byte offsets (relative to the tile's first row) of the rows
  // [row0, row0 + R) clamped to rlim - 1; the k offset is added per step.
  // NW waves share the tile.
  template <int NW>
  struct Loader {
    static constexpr int PERW = BYTES / 1024 / NW;  // loads per wave
    static_assert(PERW >= 1 && BYTES % (1024 * NW) == 0, "tile split");
    const char* base;
    int64_t ld_bytes;
    uint32_t voff[PERW];
    __device__ __forceinline__ Loader(const bf16* src, int64_t ld, int row0, int rlim, int w,
                                      int lane) {
      base = (const char*)src + (int64_t)row0 * ld * 2;
      ld_bytes = ld * 2;
#pragma unroll
      for (int m = 0; m < PERW; ++m) {
        const int q = (w * PERW + m) * 64 + lane;
        const int r = q / CPR, p = q % CPR;
        const int rr = min(r, rlim - 1 - row0);
        voff[m] = (uint32_t)((int64_t)rr * ld * 2) + (uint32_t)((p ^ f(r)) << 4);
      }
    }
    __device__ __forceinline__ void issue(char* tile, int k0, int w) const {
      const char* sb = base + (int64_t)k0 * 2;
#pragma unroll
      for (int m = 0; m < PERW; ++m) dma16_s(sb, voff[m], lds_addr(tile) + (w * PERW + m) * 1024);
    }
  };
  __device__ static __forceinline__ bf16x8 frag(const char* tile, int r, int kc) {
    return ld<bf16x8>(tile + r * RB + ((kc ^ f(r)) << 4));
  }
};

// MN-major tile: BK rows (k) x C bf16 columns.
template <int BK, int C>
struct NTile {
  static constexpr int RB = C * 2;
  static constexpr int CPR = C / 8;
  static constexpr int BYTES = BK * RB;
  static_assert(CPR >= 8, "at least 64 columns");
  // A transpose read serves 32 lanes (4 consecutive rows x 64 contiguous
  // bytes) per cycle: the rows' 4-chunk groups must land on distinct banks.
  __device__ static __forceinline__ int f(int r) { return (r & 3) << 2; }

  template <int NW>
  struct Loader {
    static constexpr int PERW = BYTES / 1024 / NW;
    static_assert(PERW >= 1 && BYTES % (1024 * NW) == 0, "tile split");
    const char* base;
    int64_t ld_bytes;
    uint32_t voff[PERW];
    __device__ __forceinline__ Loader(const bf16* src, int64_t ld, int col0, int clim, int w,
                                      int lane) {
      base = (const char*)src + (int64_t)col0 * 2;
      ld_bytes = ld * 2;
#pragma unroll
      for (int m = 0; m < PERW; ++m) {
        const int q = (w * PERW + m) * 64 + lane;
        const int r = q / CPR, p = q % CPR;
        const int c = min((p ^ f(r)) << 3, clim - 8 - col0);
        voff[m] = (uint32_t)((int64_t)r * ld * 2) + (uint32_t)(c * 2);
      }
    }
    __device__ __forceinline__ void issue(char* tile, int k0, int w) const {
      const char* sb = base + (int64_t)k0 * ld_bytes;
#pragma unroll
      for (int m = 0; m < PERW; ++m) dma16_s(sb, voff[m], lds_addr(tile) + (w * PERW + m) * 1024);
    }
  };
  // Column n0 + (lane % 32), k = 16 kk + 8 g + {0..7}.
  __device__ static __forceinline__ bf16x8 frag(const char* tile, int kk, int n0, int lane) {
    const int li = lane & 15, g = lane >> 5;
    const int col = n0 + 16 * ((lane >> 4) & 1) + 4 * (li & 3);
    const int r0 = 16 * kk + 8 * g + (li >> 2);
    const int off = ((((col >> 3) ^ f(r0)) << 4)) | (((col >> 2) & 1) << 3);  // f(r0 + 4) == f(r0)
    const char* b0 = tile + r0 * RB + off;
    const s16x4 lo =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)b0);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(b0 + 4 * RB));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
  }
};

template <bool KMAJ, int R, int BK>
struct Operand;
template <int R, int BK>
struct Operand<true, R, BK> {
  using Tile = KTile<R, BK>;
  template <int NW>
  using Loader = typename Tile::template Loader<NW>;
  // Fragment for rows r0 + (lane % 32), reduction step kk.
  __device__ static __forceinline__ bf16x8 frag(const char* t, int kk, int r0, int lane) {
    return Tile::frag(t, r0 + (lane & 31), 2 * kk + (lane >> 5));
  }
};
template <int R, int BK>
struct Operand<false, R, BK> {
  using Tile = NTile<BK, R>;
  template <int NW>
  using Loader = typename Tile::template Loader<NW>;
  __device__ static __forceinline__ bf16x8 frag(const char* t, int kk, int r0, int lane) {
    return Tile::frag(t, kk, r0, lane);
  }
};

}  // namespace gdma

// Staged epilogue, for epilogues with the value/dst interface (gemm.hpp):
// each wave writes its results, rounded to the output type, into its own LDS
// region (the stage buffers, free once every wave is past the main loop) and
// reads them back as 16-byte row pieces, so that one store instruction moves
// 16 bytes per lane instead of one 2- or 4-byte element per lane. The values
// are those of epi_apply, bit for bit.
//
// The region holds the wave's WM rows at 128 bytes each: one pass covers
// 32 JP columns of every output (JP = 2 for a single 2-byte output, else 1).
// The 16-byte pieces of row r are XOR-permuted by (r & 4): the two lane
// halves of an accumulator write (rows r and r + 4, 64 bytes each) then fall
// on different banks.
template <int WM, int FM, int FN, class Epi>
__device__ __forceinline__ void epilogue_staged(const Epi& e, const f32x16 (&acc)[FM][FN],
                                                char* region, int mw, int nw, int lane, int M,
                                                int N) {
  using U = typename Epi::Out;
  constexpr int ES = (int)sizeof(U), KO = Epi::kOuts;
  constexpr int JP = (KO * ES == 2 && FN % 2 == 0) ? 2 : 1;
  constexpr int OB = 32 * JP * ES;  // bytes of one output in a staged row
  static_assert(KO * OB <= 128, "a staged row holds 128 bytes");
  constexpr int PPO = OB / 16, VEC = 16 / ES, ITER = WM * PPO / 64;
  static_assert(WM * PPO % 64 == 0, "whole pieces per lane");
  const int lr = lane & 31, g = lane >> 5;
#pragma unroll
  for (int jp = 0; jp < FN; jp += JP) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jj = 0; jj < JP; ++jj) {
        const int col = nw + 32 * (jp + jj) + lr, cq = min(col, N - 1);
        const typename Epi::Col cv = e.col(cq);
        typename Epi::Pre pre[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
          pre[r] = e.pre(min(mw + 32 * i + acc_row(r, g), M - 1), cq, cv);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = 32 * i + acc_row(r, g);
          const float x = acc[i][jp + jj][r];
          float xp = 0.f;
          if constexpr (Epi::kPair) xp = e.paired() ? lane_xor1(x) : 0.f;
#pragma unroll
          for (int o = 0; o < KO; ++o) {
            const int b = o * OB + (32 * jj + lr) * ES;
            *(U*)(region + rl * 128 + (((b >> 4) ^ (rl & 4)) << 4) + (b & 15)) =
                from_f32<U>(e.value(o, mw + rl, col, x, xp, cv, pre[r]));
          }
        }
      }
    // LDS operations of a wave complete in order; the wait keeps the reads
    // below from being scheduled above the writes.
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int o = 0; o < KO; ++o) {
      if (!e.has(o)) continue;
#pragma unroll
      for (int it = 0; it < ITER; ++it) {
        const int idx = it * 64 + lane, rl = idx / PPO, pc = idx % PPO;
        const u32x4 val = ld<u32x4>(region + rl * 128 + (((o * PPO + pc) ^ (rl & 4)) << 4));
        const int m = mw + rl, n = nw + 32 * jp + pc * VEC;
        if (m < M && n < N) st_global((u32x4*)e.dst(o, m, n), val);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// NW waves (64 NW threads) arranged (BM / WM) x (BN / WN); LDS (STAGES stages
// of the A and B tiles) is dynamic: STAGES * (BM + BN) * BK * 2 bytes.
template <bool A_KMAJ, bool B_KMAJ, int BM, int BN, int BK, int STAGES, int WM, int WN, int NW,
          class Epi>
__global__ __launch_bounds__(64 * NW) void gemm_dma_kernel(const bf16* __restrict__ A, int64_t lda,
                                                       const bf16* __restrict__ B, int64_t ldb,
                                                       int M, int N, int K, int ksplit, Epi epi) {
  using OA = gdma::Operand<A_KMAJ, BM, BK>;
  using OB = gdma::Operand<B_KMAJ, BN, BK>;
  constexpr int ABYTES = BM * BK * 2, BBYTES = BN * BK * 2, SBYTES = ABYTES + BBYTES;
  constexpr int LOADS = SBYTES / 1024 / NW;  // direct loads per wave per stage
  constexpr int WGN = BN / WN;
  static_assert((BM / WM) * (BN / WN) == NW, "wave grid");
  constexpr int FM = WM / 32, FN = WN / 32;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;

  // Same XCD-grouped tile order as gemm_kernel.
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int nt = tiles_m * tiles_n;
  // Split-K: the grid holds ksplit copies of the tile grid, copy k summing
  // the reduction steps [k n / ksplit, (k + 1) n / ksplit) of the n = K / BK
  // steps (host: K % BK == 0, ksplit <= n).
  const int split = blockIdx.x / nt;
  int tile;
  {
    const int bid = blockIdx.x - split * nt, xcd = bid & 7, local = bid >> 3;
    const int q = nt >> 3, rem = nt & 7;
    tile = (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + local;
  }
  // Tiles in column-major order within bands of GROUP tile rows, so the
  // workgroups resident on an XCD share A rows and B columns in its L2
  // (four rows per band measured ~2 % faster than eight on these shapes).
  constexpr int GROUP = 4;
  const int group = tile / (GROUP * tiles_n);
  const int first_m = group * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (tile % (GROUP * tiles_n)) % gsz;
  const int tn = (tile % (GROUP * tiles_n)) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;
  const int wm0 = (w / WGN) * WM, wn0 = (w % WGN) * WN;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = zero16();

  const int nkt = K / BK;
  const int k0s = (int)((int64_t)split * nkt / ksplit);
  const int nk = (int)((int64_t)(split + 1) * nkt / ksplit) - k0s, kbase = k0s * BK;
  const typename OA::template Loader<NW> la(A, lda, m0, M, w, lane);
  const typename OB::template Loader<NW> lb(B, ldb, n0, N, w, lane);
  auto issue = [&](int kt) {
    char* st = smem + (kt % STAGES) * SBYTES;
    la.issue(st, kbase + kt * BK, w);
    lb.issue(st + ABYTES, kbase + kt * BK, w);
  };
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue(s);

  for (int kt = 0; kt < nk; ++kt) {
    // Stage kt is complete once at most the loads of the stages issued after
    // it remain in flight; the tail waits for everything.
    if (kt + STAGES - 2 < nk) gdma::wait_vm<(STAGES - 2) * LOADS>();
    else gdma::wait_vm<0>();
    __syncthreads();
    if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1);
    const char* As = smem + (kt % STAGES) * SBYTES;
    const char* Bs = As + ABYTES;
    // Fragments of reduction step kk + 1 are read while step kk's MFMAs run.
    constexpr int KK = BK / 16;
    bf16x8 af[2][FM], bfr[2][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) af[0][i] = OA::frag(As, 0, wm0 + 32 * i, lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) bfr[0][j] = OB::frag(Bs, 0, wn0 + 32 * j, lane);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < KK) {
#pragma unroll
        for (int i = 0; i < FM; ++i) af[cur ^ 1][i] = OA::frag(As, kk + 1, wm0 + 32 * i, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) bfr[cur ^ 1][j] = OB::frag(Bs, kk + 1, wn0 + 32 * j, lane);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mma(af[cur][i], bfr[cur][j], acc[i][j]);
    }
  }

  const int lr = lane & 31;
  const Epi e = epi_at_split(epi, split);
  if constexpr (staged_outputs<Epi>::value) {
    constexpr int VEC = 16 / (int)sizeof(typename Epi::Out);
    static_assert(NW * WM * 128 <= STAGES * SBYTES, "staging regions fit the stage buffers");
    if (N % VEC == 0 && e.vec_ok(VEC)) {
      __syncthreads();  // every wave is past its last fragment read
      epilogue_staged<WM>(e, acc, smem + w * WM * 128, m0 + wm0, n0 + wn0, lane, M, N);
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      epilogue_block<false>(e, acc[i][j], m0 + wm0 + 32 * i, n0 + wn0 + 32 * j + lr, g, M, N);
}

}  // namespace bpt
