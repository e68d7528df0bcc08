// Device helpers shared by the Lizard attention kernels (gfx950 / CDNA4).
//
// MFMA conventions used throughout (16x16 output tiles, wave of 64 lanes,
// lane = 16 * kq + r with r = lane % 16 and kq = lane / 16):
//   * operand fragment for one K = 32 step: lane (r, kq) holds the 8 values
//     k = 8*kq .. 8*kq+7 of row r (A operand: row m = r; B operand: column
//     n = r).  bf16 uses one v_mfma_f32_16x16x32_bf16; fp32 issues eight
//     v_mfma_f32_16x16x4_f32, call j pairing k-slot kq with k = 8*kq + j.
//   * accumulator: lane (r, kq) holds D[4*kq + i][r], i = 0..3.
// Both were checked on the hardware with an in-bounds probe.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lz {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { float v[8]; };

__device__ __forceinline__ f32x4 mma(const Frag<bf16> &a, const Frag<bf16> &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<float> &a, const Frag<float> &b, f32x4 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
  return c;
}

// 2^x on the transcendental unit (v_exp_f32); exponentials are written as
// exp2(fma(x, LOG2E, c)) so the base change costs no separate multiply.
constexpr float LOG2E = 1.4426950408889634f;
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// Materialise a value at this point (an empty asm that reads and writes it).  Used before a
// barrier to keep the compiler from sinking arithmetic into the next phase.
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }  // RNE
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }

template <typename T> __device__ __forceinline__ Frag<T> frag_zero() {
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = (bf16)0.0f;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = 0.0f;
  }
  return f;
}

// Fragment from 8 floats (rounded to T).
template <typename T> __device__ __forceinline__ Frag<T> frag_from(const float (&x)[8]) {
  Frag<T> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = from_f<T>(x[j]);
  return f;
}

// Buffer resource word 3 for the raw (untyped) buffer loads of gfx9-family chips: a 32-bit data
// format, so that the loads read memory (a zero format makes every access out of range).
constexpr int BUF_RSRC_WORD3 = 0x00020000;

// 8 bf16 at byte offset voff + soff of a buffer resource (reads past the resource's size return
// zeros).  soff is wave-uniform, so a wave's operand loads share one address register.
template <typename T> __device__ __forceinline__ Frag<T> buffer_load8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  static_assert(sizeof(T) == 2, "16-bit elements");
  Frag<T> f;
  f.v = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
  return f;
}

// 8 contiguous elements (16-byte aligned for bf16, 32-byte for fp32).
template <typename T> __device__ __forceinline__ Frag<T> load8(const T *p) {
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
    f.v = *reinterpret_cast<const bf16x8 *>(p);
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) { f.v[j] = a[j]; f.v[4 + j] = b[j]; }
  }
  return f;
}

// 4 contiguous elements at p0 (slots 0..3) and 4 at p1 (slots 4..7).
template <typename T> __device__ __forceinline__ Frag<T> load4x2(const T *p0, const T *p1) {
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
    const bf16x4 a = *reinterpret_cast<const bf16x4 *>(p0);
    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(p1);
#pragma unroll
    for (int j = 0; j < 4; ++j) { f.v[j] = a[j]; f.v[4 + j] = b[j]; }
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p0);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p1);
#pragma unroll
    for (int j = 0; j < 4; ++j) { f.v[j] = a[j]; f.v[4 + j] = b[j]; }
  }
  return f;
}

// 8 / 4 contiguous elements converted to float.
template <typename T> __device__ __forceinline__ void load8f(const T *p, float (&x)[8]) {
  if constexpr (sizeof(T) == 2) {
    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = (float)a[j];
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) { x[j] = a[j]; x[4 + j] = b[j]; }
  }
}
template <typename T> __device__ __forceinline__ void load4f(const T *p, float (&x)[4]) {
  if constexpr (sizeof(T) == 2) {
    const bf16x4 a = *reinterpret_cast<const bf16x4 *>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = (float)a[j];
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = a[j];
  }
}

// Store 4 floats as 4 contiguous T.
template <typename T> __device__ __forceinline__ void store4(T *p, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 2) {
    bf16x4 v;
    v[0] = (bf16)a; v[1] = (bf16)b; v[2] = (bf16)c; v[3] = (bf16)d;
    *reinterpret_cast<bf16x4 *>(p) = v;
  } else {
    f32x4 v = {a, b, c, d};
    *reinterpret_cast<f32x4 *>(p) = v;
  }
}

// Cross-lane reductions without the LDS crossbar: DPP moves inside each row of
// 16 lanes, and the gfx950 permlane swaps across rows.  permlane16_swap(x, x)
// yields, per lane l, the pair {x[l], x[l ^ 16]} (in either order) and
// permlane32_swap(x, x) the pair {x[l], x[l ^ 32]}, so a symmetric operation
// on the pair reduces across the rows; every lane gets the same bits.
template <int CTRL> __device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <- 7 - i within 8
constexpr int DPP_MIRROR = 0x140;      // lane i <- 15 - i within 16

__device__ __forceinline__ float pair16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// max / sum over the 16 lanes of a row
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_f<DPP_XOR1>(x));
  x = fmaxf(x, dpp_f<DPP_XOR2>(x));
  x = fmaxf(x, dpp_f<DPP_HALF_MIRROR>(x));
  return fmaxf(x, dpp_f<DPP_MIRROR>(x));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f<DPP_XOR1>(x);
  x += dpp_f<DPP_XOR2>(x);
  x += dpp_f<DPP_HALF_MIRROR>(x);
  return x + dpp_f<DPP_MIRROR>(x);
}
// max / sum over the four lanes that share lane % 16 (a column of an MFMA tile)
__device__ __forceinline__ float wave_max_cols(float x) { return pair32_max(pair16_max(x)); }
__device__ __forceinline__ float wave_sum_cols(float x) { return pair32_sum(pair16_sum(x)); }
__device__ __forceinline__ float wave_max_all(float x) { return wave_max_cols(row_max16(x)); }

}  // namespace lz
