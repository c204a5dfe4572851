// Device-side building blocks shared by the layer's gfx950 kernels: storage
// types, 32x32 MFMA tiles, vector loads and lane-layout helpers.
//
// MFMA tile convention used everywhere (wave64, 32x32 output tile):
//   * operand A (rows m of the output): lane l holds row m = l % 32 and the 8
//     reduction indices of "half" g = l / 32 of a 16-wide reduction chunk;
//   * operand B (columns n of the output): lane l holds column n = l % 32 and
//     the same 8 reduction indices of half g;
//   * accumulator C (16 fp32 per lane): lane l holds column n = l % 32 and
//     rows (r / 4) * 8 + g * 4 + (r % 4), r = 0..15.
// Only the A/B pairing of reduction indices matters for the result, so a
// kernel may feed any fixed permutation of the 16 reduction indices as long
// as A and B use the same one.
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bpt {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Eight storage elements: one MFMA operand fragment of a 16-wide chunk.
template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// acc += A * B on a 32x32 tile over one 16-wide reduction chunk.
__device__ __forceinline__ f32x16 mma(const bf16x8& a, const bf16x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma(const f32x8& a, const f32x8& b, f32x16 c) {
  // fp32: eight k=2 steps; element e of both halves forms reduction pair e.
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
  return c;
}

// Row of accumulator register r for lane half g.
__device__ __forceinline__ int acc_row(int r, int g) { return (r >> 2) * 8 + g * 4 + (r & 3); }

// 16-byte and 8-byte vector memory helpers (generic address space).
template <typename V>
__device__ __forceinline__ V ld(const void* p) { return *reinterpret_cast<const V*>(p); }
template <typename V>
__device__ __forceinline__ void st(void* p, const V& v) { *reinterpret_cast<V*>(p) = v; }

// Load the 8 contiguous elements at p as a fragment.
__device__ __forceinline__ bf16x8 ld_frag(const bf16* p) { return ld<bf16x8>(p); }
__device__ __forceinline__ f32x8 ld_frag(const float* p) {
  f32x4 a = ld<f32x4>(p), b = ld<f32x4>(p + 4);
  f32x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}
// Load 4 + 4 elements from p0 and p1 as one fragment (elements 0-3, 4-7).
__device__ __forceinline__ bf16x8 ld_frag_split(const bf16* p0, const bf16* p1) {
  u32x2 a = ld<u32x2>(p0), b = ld<u32x2>(p1);
  u32x4 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  return __builtin_bit_cast(bf16x8, r);
}
__device__ __forceinline__ f32x8 ld_frag_split(const float* p0, const float* p1) {
  f32x4 a = ld<f32x4>(p0), b = ld<f32x4>(p1);
  f32x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// Fragment from 8 fp32 values (rounded to the storage type).
template <typename T> __device__ __forceinline__ typename Frag<T>::type pack_frag(const float* v);
template <> __device__ __forceinline__ bf16x8 pack_frag<bf16>(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)v[e];
  return r;
}
template <> __device__ __forceinline__ f32x8 pack_frag<float>(const float* v) {
  f32x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = v[e];
  return r;
}

// 4 x VEC sub-block transpose: in[i] holds VEC elements of reduction row i;
// out[j] receives the 4 reduction elements of output row j.
__device__ __forceinline__ void transpose_4xvec(const u32x4 in[4], u32x2 out[8]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    out[2 * w][0] = (in[0][w] & 0xFFFFu) | (in[1][w] << 16);
    out[2 * w][1] = (in[2][w] & 0xFFFFu) | (in[3][w] << 16);
    out[2 * w + 1][0] = (in[0][w] >> 16) | (in[1][w] & 0xFFFF0000u);
    out[2 * w + 1][1] = (in[2][w] >> 16) | (in[3][w] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void transpose_4xvec(const u32x4 in[4], u32x4 out[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[j][0] = in[0][j]; out[j][1] = in[1][j]; out[j][2] = in[2][j]; out[j][3] = in[3][j];
  }
}

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, kWave); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum of the 32 bf16 values of v[0..3]: sixteen v_dot2c_f32_bf16 with
// (1.0, 1.0) accumulating into one register. Written as inline asm (the
// builtin's vector operands were observed to be mis-selected, one dword used
// for all four products), in one block that ends with three wait states: a
// different VALU instruction may read a dot-product result only three wait
// states after it is written, and the compiler's hazard tracking does not
// see into inline assembly.
__device__ __forceinline__ float row_sum_bf16x32(const bf16x8 (&v)[4]) {
  const u32x4 a = __builtin_bit_cast(u32x4, v[0]), b = __builtin_bit_cast(u32x4, v[1]);
  const u32x4 c = __builtin_bit_cast(u32x4, v[2]), d = __builtin_bit_cast(u32x4, v[3]);
  float acc = 0.f;
  asm("v_dot2c_f32_bf16 %0, 0x3f803f80, %1\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %2\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %3\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %4\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %5\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %6\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %7\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %8\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %9\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %10\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %11\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %12\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %13\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %14\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %15\n\t"
      "v_dot2c_f32_bf16 %0, 0x3f803f80, %16\n\t"
      "s_nop 2"
      : "+v"(acc)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]),
        "v"(c[0]), "v"(c[1]), "v"(c[2]), "v"(c[3]), "v"(d[0]), "v"(d[1]), "v"(d[2]), "v"(d[3]));
  return acc;
}

// ---------------------------------------------------------------- direct loads
// global_load_lds_dwordx4: 16 bytes per lane from global memory straight into
// LDS at M0 + 16 * lane. Issued through inline asm so that the compiler's
// wait-count pass does not treat every later LDS read as dependent on the
// load (it cannot tell the tile being filled from the tiles being read, and
// would wait for all outstanding loads before the first LDS read after it).
// Callers therefore wait for these loads themselves (s_waitcnt vmcnt) before
// the barrier that publishes a tile. M0 is saved and restored around the
// load; one wait state separates the M0 write from the load.
//
// dma16_s: wave-uniform 64-bit base (SGPRs) + per-lane 32-bit byte offset.
// dma16_v: per-lane 64-bit address.
// lds: wave-uniform LDS byte address of the 64 x 16-byte destination block.
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(sbase)
      : "memory");
}
__device__ __forceinline__ void dma16_v(const void* addr, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(addr)
      : "memory");
}

// LDS byte address of a shared-memory object.
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
  return (uint32_t)(size_t)((const __attribute__((address_space(3))) char*)p);
}

}  // namespace bpt
