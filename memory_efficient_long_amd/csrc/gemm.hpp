// MFMA GEMM for gfx950 with fused epilogues.
//
//   C[m, n] = sum_k A(m, k) * B(n, k)          (fp32 accumulation)
//
// Operand storage (row-major in memory):
//   A_KMAJ: A(m, k) = A[m * lda + k]   (activations, K contiguous)
//   else  : A(m, k) = A[k * lda + m]   (M contiguous; e.g. X^T for dW = X^T dY)
//   B_KMAJ: B(n, k) = B[n * ldb + k]   (e.g. W for dX = dY W^T)
//   else  : B(n, k) = B[k * ldb + n]   (e.g. a weight [in, out] for y = x W)
//
// Tiles are staged in LDS K-contiguous (padded by 16 B per row). An
// MN-contiguous operand is loaded as 4(k) x 8(m) bf16 sub-blocks with 16-byte
// global loads and transposed in registers before the LDS store, so every
// layout the layer needs (forward x W, backward dY W^T and X^T dY) runs on the
// same MFMA inner loop without separate transpose passes.
//
// Workgroup: 256 threads = 4 waves, each owning a (BM/2) x (BN/2) block of
// 32 x 32 MFMA tiles (the layer uses 128 x 128 tiles: two workgroups per CU). Global loads of
// the next K step are issued before the current step's MFMAs (register
// prefetch, LDS double buffer).
#pragma once

#include "device_common.hpp"

namespace bpt {

// ----------------------------------------------------------------- activations
__device__ __forceinline__ float act_relu(float a) { return a > 0.f ? a : 0.f; }
// erf(x) for x >= 0 together with exp(-x^2), by the rational approximation
// of Abramowitz & Stegun, Handbook of Mathematical Functions, 7.1.26:
// erf(x) = 1 - (a1 t + ... + a5 t^5) exp(-x^2), t = 1 / (1 + p x), absolute
// error <= 1.5e-7 -- far below the bf16 rounding of the GEMM outputs it
// feeds, at a fraction of the cost of a full-precision erff.
__device__ __forceinline__ float erf_as(float x, float& ex2) {
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.f));
  const float poly =
      t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f),
                       -0.284496736f),
               0.254829592f);
  ex2 = fast_exp2(-x * x * 1.4426950408889634f);
  return 1.f - poly * ex2;
}
// GELU with the exact (erf) form: 0.5 a (1 + erf(a / sqrt 2)).
__device__ __forceinline__ float act_gelu(float a) {
  float ex2;
  const float e = erf_as(fabsf(a) * 0.70710678118654752f, ex2);
  return 0.5f * a * (1.f + copysignf(e, a));
}
// d GELU / da = Phi(a) + a phi(a); exp(-(a / sqrt 2)^2) is phi's exponential.
__device__ __forceinline__ float act_gelu_grad(float a) {
  float ex2;
  const float e = erf_as(fabsf(a) * 0.70710678118654752f, ex2);
  return 0.5f * (1.f + copysignf(e, a)) + a * 0.39894228040143268f * ex2;
}
// 1 / (1 + e^-a) with the hardware exp2 and reciprocal (about 1 ulp each).
__device__ __forceinline__ float sigmoidf_(float a) {
  return __builtin_amdgcn_rcpf(1.f + fast_exp2(-a * 1.4426950408889634f));
}

enum ActKind { ACT_RELU = 0, ACT_GELU = 1 };

// Value of lane ^ 1 (the neighbouring accumulator column): a DPP quad
// permutation [1, 0, 3, 2], a single VALU move (every source lane is valid,
// so no old value is kept: no extra move to initialise the destination).
__device__ __forceinline__ float lane_xor1(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
}

// ----------------------------------------------------------------- epilogues
// Each epilogue is applied to one 32 x 32 accumulator block of a lane (one
// column, 16 rows) in three steps: col(n) loads what depends on the column
// only (a bias), pre(m, n, col) gathers each element's other inputs
// (residual, previous value, ...) for all 16 rows, then the values are
// computed and stored. Gathering first, unconditionally from clamped indices, matters
// on this GPU: vector-memory loads and stores share one in-order counter, so
// a load issued after stores -- or inside its own branch -- cannot be waited
// for without also waiting for everything before it. v is the fp32
// accumulator value; vp, when kPair, the value of column n ^ 1 in the same
// row (used by the RoPE rotation).
//
// The computing and storing are split: an epilogue has kOuts outputs of
// element type Out; value(o, ...) is what output o holds at (m, n) (before
// rounding to Out) and dst(o, m, n) its address, with 16 / sizeof(Out)
// consecutive columns (from a multiple of that count) contiguous in memory
// whenever vec_ok(16 / sizeof(Out)) holds; has(o) says whether output o is
// written at all. epi_apply stores one element; the direct-load GEMM also
// stores whole 16-byte row pieces (see epilogue_staged), with the same values.

__device__ __forceinline__ bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// a, b or c (b when b1, c when also b2) by address arithmetic: a select among
// neighbouring pointer fields of an epilogue becomes a load at a computed
// offset, which keeps the whole epilogue object in scratch memory.
template <typename P>
__device__ __forceinline__ P* pick3(P* a, P* b, P* c, bool b1, bool b2) {
  const uintptr_t ua = (uintptr_t)a, ub = (uintptr_t)b, uc = (uintptr_t)c;
  return (P*)(ua + (b1 ? ub - ua : 0) + (b2 ? uc - ub : 0));
}

// Epilogues whose outputs the direct-load GEMM stages through LDS: those with
// the value/dst interface that ask for it (kStaged) and have 2-byte outputs
// (a half-wave's fp32 row segment, 32 columns, is already a whole 128-byte
// line; staging it measured slower).
template <class E, class = void>
struct staged_outputs : std::false_type {};
template <class E>
struct staged_outputs<E, std::void_t<decltype(E::kOuts)>>
    : std::bool_constant<E::kStaged && sizeof(typename E::Out) == 2> {};

// Store through a global-memory pointer (an output address computed by
// integer arithmetic would otherwise be stored to as a generic one).
template <typename V>
__device__ __forceinline__ void st_global(V* p, V v) {
  *(__attribute__((address_space(1))) V*)p = v;
}

template <class Epi>
__device__ __forceinline__ void epi_apply(const Epi& e, int m, int n, float v, float vp,
                                          const typename Epi::Col& c,
                                          const typename Epi::Pre& p) {
#pragma unroll
  for (int o = 0; o < Epi::kOuts; ++o)
    if (e.has(o)) st_global(e.dst(o, m, n), from_f32<typename Epi::Out>(e.value(o, m, n, v, vp, c, p)));
}

// out = alpha * v (+ bias[n]) (+ out if accumulate)
template <typename T, typename OutT>
struct EpiOut {
  OutT* out; int64_t ldo; const T* bias; float alpha; int accumulate;
  static constexpr bool kPair = false;
  using Out = OutT;
  static constexpr int kOuts = 1;
  static constexpr bool kStaged = true;
  struct Col { float b; };
  struct Pre { float o; };
  __device__ __forceinline__ Col col(int n) const { return {bias ? to_f32(bias[n]) : 0.f}; }
  __device__ __forceinline__ Pre pre(int m, int n, const Col&) const {
    return {accumulate ? to_f32(out[(int64_t)m * ldo + n]) : 0.f};
  }
  __device__ __forceinline__ bool has(int) const { return true; }
  __device__ __forceinline__ bool vec_ok(int vec) const { return al16(out) && ldo % vec == 0; }
  __device__ __forceinline__ float value(int, int, int, float v, float, const Col& c,
                                         const Pre& p) const {
    return fmaf(alpha, v, c.b + p.o);
  }
  __device__ __forceinline__ Out* dst(int, int m, int n) const { return out + (int64_t)m * ldo + n; }
};

// out_k[m, n - start_k] (+)= v for the three column segments [0, c1),
// [c1, c2), [c2, N) (start_k = 0, c1, c2) of the product, each written into
// its own column range of an fp32 matrix with row stride ldo: the weight
// gradient of a head chunk, whose Q, K and V columns are apart in W_qkv.
template <typename T>
struct EpiOut3 {
  float* out0; float* out1; float* out2; int64_t ldo; int c1, c2; int accumulate;
  static constexpr bool kPair = false;
  using Out = float;
  static constexpr int kOuts = 1;
  static constexpr bool kStaged = true;
  struct Col { float* dst; };
  struct Pre { float o; };
  __device__ __forceinline__ float* seg(int n) const {
    return pick3(out0, out1, out2, n >= c1, n >= c2) + (n < c1 ? n : (n < c2 ? n - c1 : n - c2));
  }
  __device__ __forceinline__ Col col(int n) const { return {seg(n)}; }
  __device__ __forceinline__ Pre pre(int m, int, const Col& c) const {
    return {accumulate ? c.dst[(int64_t)m * ldo] : 0.f};
  }
  __device__ __forceinline__ bool has(int) const { return true; }
  __device__ __forceinline__ bool vec_ok(int vec) const {
    return al16(out0) && al16(out1) && al16(out2) && ldo % vec == 0 && c1 % vec == 0 &&
           c2 % vec == 0;
  }
  __device__ __forceinline__ float value(int, int, int, float v, float, const Col&,
                                         const Pre& p) const {
    return v + p.o;
  }
  __device__ __forceinline__ Out* dst(int, int m, int n) const { return seg(n) + (int64_t)m * ldo; }
};

// Split-K partial product: copy k of the split grid writes its raw fp32 sum
// to out + k split_stride ([M, ldo] each); splitk_reduce_kernel then applies
// the real epilogue to the sum of the copies.
struct EpiPart {
  float* out; int64_t ldo; int64_t split_stride;
  static constexpr bool kPair = false;
  using Out = float;
  static constexpr int kOuts = 1;
  static constexpr bool kStaged = true;
  struct Col {};
  struct Pre {};
  __device__ __forceinline__ Col col(int) const { return {}; }
  __device__ __forceinline__ Pre pre(int, int, const Col&) const { return {}; }
  __device__ __forceinline__ bool has(int) const { return true; }
  __device__ __forceinline__ bool vec_ok(int vec) const {
    return al16(out) && ldo % vec == 0 && split_stride % vec == 0;
  }
  __device__ __forceinline__ float value(int, int, int, float v, float, const Col&,
                                         const Pre&) const {
    return v;
  }
  __device__ __forceinline__ Out* dst(int, int m, int n) const { return out + (int64_t)m * ldo + n; }
};
template <class Epi>
__device__ __forceinline__ Epi epi_at_split(const Epi& e, int) { return e; }
__device__ __forceinline__ EpiPart epi_at_split(const EpiPart& e, int k) {
  EpiPart r = e;
  r.out += k * e.split_stride;
  return r;
}

// out = Epi(sum over k < nsplit of part[k, m, n]), one element per thread, the
// copies summed in order (deterministic).
template <class Epi>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int nsplit, int M, int N, Epi epi) {
  const int64_t mn = (int64_t)M * N;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= mn) return;
  const int m = (int)(i / N), n = (int)(i - (int64_t)m * N);
  float v = 0.f;
  for (int k = 0; k < nsplit; ++k) v += part[k * mn + i];
  const typename Epi::Col c = epi.col(n);
  const typename Epi::Pre p = epi.pre(m, n, c);
  epi_apply(epi, m, n, v, 0.f, c, p);
}

// Q, K and V projections of all heads in one GEMM (columns [0, c1) -> q,
// [c1, c2) -> k, [c2, N) -> v; c1, c2 multiples of D): + bias, RoPE on the
// q and k columns, scattered to head-major [heads, s, D] buffers. The q
// columns are also multiplied by qmul (log2(e)/sqrt(D)) before rounding, so
// the attention kernels' products Q K^T are scores in base-2 units and need
// no per-element scaling. Everything that depends on the column only (bias,
// destination, rotation role, factor) is resolved once per lane in col();
// each element then costs its arithmetic and a store.
template <typename T>
struct EpiQKV3 {
  T* q; T* k; T* v; int64_t head_stride; int D; const T* bias; const float2* rope; int c1, c2;
  float qmul;
  static constexpr bool kPair = true;
  using Out = T;
  static constexpr int kOuts = 1;
  static constexpr bool kStaged = true;
  struct Col { float b, bp, mul; int rc, rot; };  // rot: 0 none, 1 even, 2 odd member
  struct Pre { float2 cs; };
  __device__ __forceinline__ Col col(int n) const {
    const int nn = n < c1 ? n : (n < c2 ? n - c1 : n - c2);
    const int dd = nn % D;
    Col c;
    c.b = bias ? to_f32(bias[n]) : 0.f;
    c.bp = bias ? to_f32(bias[n ^ 1]) : 0.f;
    c.mul = n < c1 ? qmul : 1.f;
    c.rc = dd >> 1;
    c.rot = rope && n < c2 ? 1 + (dd & 1) : 0;
    return c;
  }
  // Branches only on `rope` (uniform across the wave); the per-lane role is
  // applied with selects.
  __device__ __forceinline__ bool paired() const { return rope != nullptr; }
  // The rotation entry is loaded for every column when RoPE is on (v columns
  // ignore it): the address is valid for any column, and no per-lane branch
  // guards the load.
  __device__ __forceinline__ Pre pre(int m, int, const Col& c) const {
    if (!rope) return {{1.f, 0.f}};
    return {rope[(int64_t)m * (D / 2) + c.rc]};
  }
  __device__ __forceinline__ bool has(int) const { return true; }
  __device__ __forceinline__ bool vec_ok(int vec) const {
    return al16(q) && al16(k) && al16(this->v) && head_stride % vec == 0 && D % vec == 0;
  }
  __device__ __forceinline__ float value(int, int, int, float val, float vp, const Col& c,
                                         const Pre& p) const {
    val += c.b;
    if (rope) {
      vp += c.bp;
      const float r = c.rot == 2 ? (vp * p.cs.y + val * p.cs.x) : (val * p.cs.x - vp * p.cs.y);
      val = c.rot ? r : val;
    }
    return val * c.mul;
  }
  __device__ __forceinline__ Out* dst(int, int m, int n) const {
    const int nn = n < c1 ? n : (n < c2 ? n - c1 : n - c2);
    const int head = nn / D, dd = nn - head * D;
    return pick3(q, k, this->v, n >= c1, n >= c2) + (int64_t)head * head_stride +
           (int64_t)m * D + dd;
  }
};

// out = v + bias[n] + res[m, n]
template <typename T, typename ResT, typename OutT>
struct EpiResid {
  OutT* out; int64_t ldo; const ResT* res; int64_t ldr; const T* bias;
  static constexpr bool kPair = false;
  using Out = OutT;
  static constexpr int kOuts = 1;
  static constexpr bool kStaged = true;
  struct Col { float b; };
  struct Pre { float r; };
  __device__ __forceinline__ Col col(int n) const { return {bias ? to_f32(bias[n]) : 0.f}; }
  __device__ __forceinline__ Pre pre(int m, int n, const Col&) const {
    return {to_f32(res[(int64_t)m * ldr + n])};
  }
  __device__ __forceinline__ bool has(int) const { return true; }
  __device__ __forceinline__ bool vec_ok(int vec) const { return al16(out) && ldo % vec == 0; }
  __device__ __forceinline__ float value(int, int, int, float v, float, const Col& c,
                                         const Pre& p) const {
    return v + c.b + p.r;
  }
  __device__ __forceinline__ Out* dst(int, int m, int n) const { return out + (int64_t)m * ldo + n; }
};

// a = v + bias[n]; optionally keep a; u = act(a)
template <typename T>
struct EpiAct {
  T* u; T* a_keep; int64_t ldo; const T* bias; int act;
  static constexpr bool kPair = false;
  using Out = T;
  static constexpr int kOuts = 2;  // u, then a (kept when a_keep is given)
  static constexpr bool kStaged = true;
  struct Col { float b; };
  struct Pre {};
  __device__ __forceinline__ Col col(int n) const { return {bias ? to_f32(bias[n]) : 0.f}; }
  __device__ __forceinline__ Pre pre(int, int, const Col&) const { return {}; }
  __device__ __forceinline__ bool has(int o) const { return o == 0 || a_keep != nullptr; }
  __device__ __forceinline__ bool vec_ok(int vec) const {
    return al16(u) && (!a_keep || al16(a_keep)) && ldo % vec == 0;
  }
  __device__ __forceinline__ float value(int o, int, int, float v, float, const Col& c,
                                         const Pre&) const {
    v += c.b;
    return o == 1 ? v : (act == ACT_RELU ? act_relu(v) : act_gelu(v));
  }
  __device__ __forceinline__ Out* dst(int o, int m, int n) const {
    return (o == 0 ? u : a_keep) + (int64_t)m * ldo + n;
  }
};

// SwiGLU up projection: u = silu(gate[m, n]) * v; optionally keep v.
template <typename T>
struct EpiSwiUp {
  T* u; T* up_keep; const T* gate; int64_t ldo;
  static constexpr bool kPair = false;
  using Out = T;
  static constexpr int kOuts = 2;  // u, then the up projection (kept when up_keep is given)
  static constexpr bool kStaged = true;
  struct Col {};
  struct Pre { float g; };
  __device__ __forceinline__ Col col(int) const { return {}; }
  __device__ __forceinline__ Pre pre(int m, int n, const Col&) const {
    return {to_f32(gate[(int64_t)m * ldo + n])};
  }
  __device__ __forceinline__ bool has(int o) const { return o == 0 || up_keep != nullptr; }
  __device__ __forceinline__ bool vec_ok(int vec) const {
    return al16(u) && (!up_keep || al16(up_keep)) && ldo % vec == 0;
  }
  __device__ __forceinline__ float value(int o, int, int, float v, float, const Col&,
                                         const Pre& p) const {
    return o == 1 ? v : p.g * sigmoidf_(p.g) * v;
  }
  __device__ __forceinline__ Out* dst(int o, int m, int n) const {
    return (o == 0 ? u : up_keep) + (int64_t)m * ldo + n;
  }
};

// da = v * act'(a[m, n])
template <typename T>
struct EpiActGrad {
  T* da; const T* a; int64_t ldo; int act;
  static constexpr bool kPair = false;
  using Out = T;
  static constexpr int kOuts = 1;
  static constexpr bool kStaged = true;
  struct Col {};
  struct Pre { float x; };
  __device__ __forceinline__ Col col(int) const { return {}; }
  __device__ __forceinline__ Pre pre(int m, int n, const Col&) const {
    return {to_f32(a[(int64_t)m * ldo + n])};
  }
  __device__ __forceinline__ bool has(int) const { return true; }
  __device__ __forceinline__ bool vec_ok(int vec) const { return al16(da) && ldo % vec == 0; }
  __device__ __forceinline__ float value(int, int, int, float v, float, const Col&,
                                         const Pre& p) const {
    const float gr = act == ACT_RELU ? (p.x > 0.f ? 1.f : 0.f) : act_gelu_grad(p.x);
    return v * gr;
  }
  __device__ __forceinline__ Out* dst(int, int m, int n) const { return da + (int64_t)m * ldo + n; }
};

// SwiGLU backward from du = v: d gate = du * up * s(g) (1 + g (1 - s(g))),
// d up = du * g * s(g).
template <typename T>
struct EpiSwiGrad {
  T* dgate; T* dup; const T* gate; const T* up; int64_t ldo;
  static constexpr bool kPair = false;
  using Out = T;
  static constexpr int kOuts = 2;  // d gate, d up
  // Staging measured slower here (two gathered inputs, two outputs).
  static constexpr bool kStaged = false;
  struct Col {};
  struct Pre { float g, u; };
  __device__ __forceinline__ Col col(int) const { return {}; }
  __device__ __forceinline__ Pre pre(int m, int n, const Col&) const {
    const int64_t i = (int64_t)m * ldo + n;
    return {to_f32(gate[i]), to_f32(up[i])};
  }
  __device__ __forceinline__ bool has(int) const { return true; }
  __device__ __forceinline__ bool vec_ok(int vec) const {
    return al16(dgate) && al16(dup) && ldo % vec == 0;
  }
  __device__ __forceinline__ float value(int o, int, int, float v, float, const Col&,
                                         const Pre& p) const {
    const float sg = sigmoidf_(p.g);
    return o == 0 ? v * p.u * sg * (1.f + p.g * (1.f - sg)) : v * p.g * sg;
  }
  __device__ __forceinline__ Out* dst(int o, int m, int n) const {
    return (o == 0 ? dgate : dup) + (int64_t)m * ldo + n;
  }
};

// Epilogue of one 32 x 32 accumulator block (rows m0 + acc_row(r, g), column
// col of this lane). Inputs are gathered from indices clamped into the
// matrix (M, N > 0), so the loads need no branches; only stores are guarded.
template <bool EVEN, class Epi>
__device__ __forceinline__ void epilogue_block(const Epi& epi, const f32x16& acc, int m0, int col,
                                               int g, int M, int N) {
  const int cq = EVEN ? col : min(col, N - 1);
  const typename Epi::Col cv = epi.col(cq);
  typename Epi::Pre pre[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = m0 + acc_row(r, g);
    pre[r] = epi.pre(EVEN ? row : min(row, M - 1), cq, cv);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = m0 + acc_row(r, g);
    const float v = acc[r];
    float vp = 0.f;
    if constexpr (Epi::kPair) vp = epi.paired() ? lane_xor1(v) : 0.f;
    if (EVEN || (row < M && col < N)) epi_apply(epi, row, col, v, vp, cv, pre[r]);
  }
}

// ----------------------------------------------------------------- tile loaders
// Loads one operand tile (R rows x BK reduction) into registers and stores it
// K-contiguous into LDS (rows padded by 16 bytes). K-major sources are read as
// 16-byte row chunks; MN-major sources as 4(k) x 16-byte sub-blocks that are
// transposed in registers. EVEN skips the bounds checks (every tile is full).
template <typename T, bool KMAJ, int R, int BK, bool EVEN>
struct TileLoader {
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int LDK = BK + VEC;
  static constexpr int CHUNKS = R * BK / VEC;            // 16-byte chunks per tile
  static constexpr int PER = CHUNKS / 256;               // per thread
  static_assert(CHUNKS % 1024 == 0, "tile must be a multiple of 4 x 16 B per thread");
  u32x4 reg[PER];

  __device__ __forceinline__ void load(const T* __restrict__ src, int64_t ldm, int row0, int rlim,
                                       int k0, int K, int tid) {
    if constexpr (KMAJ) {
      constexpr int CPR = BK / VEC;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int c = tid + 256 * i;
        const int r = c / CPR, kc = (c % CPR) * VEC;
        const int gr = row0 + r, gk = k0 + kc;
        if (EVEN || (gr < rlim && gk < K)) reg[i] = ld<u32x4>(src + (int64_t)gr * ldm + gk);
        else reg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    } else {
      constexpr int KB = BK / 4;
#pragma unroll
      for (int i = 0; i < PER / 4; ++i) {
        const int sb = tid + 256 * i;
        const int kb = sb % KB, rb = sb / KB;
        const int gr = row0 + rb * VEC;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int gk = k0 + 4 * kb + j;
          if (EVEN || (gr < rlim && gk < K)) reg[4 * i + j] = ld<u32x4>(src + (int64_t)gk * ldm + gr);
          else reg[4 * i + j] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  }

  __device__ __forceinline__ void store(T* tile, int tid) const {
    if constexpr (KMAJ) {
      constexpr int CPR = BK / VEC;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int c = tid + 256 * i;
        const int r = c / CPR, kc = (c % CPR) * VEC;
        st<u32x4>(tile + r * LDK + kc, reg[i]);
      }
    } else {
      constexpr int KB = BK / 4;
#pragma unroll
      for (int i = 0; i < PER / 4; ++i) {
        const int sb = tid + 256 * i;
        const int kb = sb % KB, rb = sb / KB;
        if constexpr (sizeof(T) == 2) {
          u32x2 out[8];
          transpose_4xvec(&reg[4 * i], out);
#pragma unroll
          for (int j = 0; j < 8; ++j) st<u32x2>(tile + (rb * 8 + j) * LDK + 4 * kb, out[j]);
        } else {
          u32x4 out[4];
          transpose_4xvec(&reg[4 * i], out);
#pragma unroll
          for (int j = 0; j < 4; ++j) st<u32x4>(tile + (rb * 4 + j) * LDK + 4 * kb, out[j]);
        }
      }
    }
  }
};

// ----------------------------------------------------------------- kernel
// BM x BN output tile per workgroup of 4 waves arranged (BM/WM) x (BN/WN);
// each wave owns WM x WN as (WM/32) x (WN/32) MFMA tiles.
template <typename T, bool A_KMAJ, bool B_KMAJ, int BM, int BN, int BK, int WM, int WN, bool EVEN,
          class Epi>
__global__ __launch_bounds__(256) void gemm_kernel(const T* __restrict__ A, int64_t lda,
                                                   const T* __restrict__ B, int64_t ldb, int M,
                                                   int N, int K, Epi epi) {
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int LDK = BK + VEC;
  constexpr int WGN = BN / WN;
  static_assert((BM / WM) * (BN / WN) == 4, "4 waves per workgroup");
  constexpr int FM = WM / 32, FN = WN / 32;
  __shared__ __attribute__((aligned(16))) T smem[2][(BM + BN) * LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, g = lane >> 5;

  // Tile order: each XCD (workgroups are dealt round-robin over 8) owns a
  // contiguous range of tiles, walked in groups of 8 tile-rows so the
  // workgroups resident on one XCD share A and B tiles in its L2.
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int nt = tiles_m * tiles_n;
  int tile;
  {
    const int bid = blockIdx.x, xcd = bid & 7, local = bid >> 3;
    const int q = nt >> 3, rem = nt & 7;
    tile = (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + local;
  }
  constexpr int GROUP = 8;
  const int group = tile / (GROUP * tiles_n);
  const int first_m = group * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (tile % (GROUP * tiles_n)) % gsz;
  const int tn = (tile % (GROUP * tiles_n)) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;
  const int wm0 = (w / WGN) * WM, wn0 = (w % WGN) * WN;

  TileLoader<T, A_KMAJ, BM, BK, EVEN> la;
  TileLoader<T, B_KMAJ, BN, BK, EVEN> lb;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = zero16();

  const int nk = (K + BK - 1) / BK;
  if (nk > 0) {
    la.load(A, lda, m0, M, 0, K, tid);
    lb.load(B, ldb, n0, N, 0, K, tid);
    la.store(smem[0], tid);
    lb.store(smem[0] + BM * LDK, tid);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) {
      la.load(A, lda, m0, M, (kt + 1) * BK, K, tid);
      lb.load(B, ldb, n0, N, (kt + 1) * BK, K, tid);
    }
    const T* As = smem[buf];
    const T* Bs = smem[buf] + BM * LDK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      typename Frag<T>::type af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = ld_frag(As + (wm0 + 32 * i + lr) * LDK + 16 * kk + 8 * g);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = ld_frag(Bs + (wn0 + 32 * j + lr) * LDK + 16 * kk + 8 * g);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mma(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) {
      la.store(smem[buf ^ 1], tid);
      lb.store(smem[buf ^ 1] + BM * LDK, tid);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      epilogue_block<EVEN>(epi, acc[i][j], m0 + wm0 + 32 * i, n0 + wn0 + 32 * j + lr, g, M, N);
}

}  // namespace bpt
