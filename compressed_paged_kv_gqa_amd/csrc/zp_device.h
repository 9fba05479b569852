// Device helpers for the gfx950 kernels of libzp: bf16 conversion, 16-byte
// vector access, wavefront reductions on DPP / swizzle, and the launch-side
// error helpers shared by the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zp.h"

namespace zp {

// bf16 is carried as its raw 16-bit pattern.
using bf16_t = uint16_t;

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// float -> bf16, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<bf16_t>(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }

// Unpacks a 16-byte vector into fp32 values: 8 for bf16, 4 for fp32.
template <typename T>
struct Vec16;
template <>
struct Vec16<bf16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void unpack(const uint4& v, float* f) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  }
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// 16-byte load marked non-temporal: for data streamed once (K/V pages in
// decode). On MI355X such loads sustain ~88% of HBM peak against ~78% for
// ordinary loads (measured with a streaming-read probe).
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  typedef unsigned int u4v __attribute__((ext_vector_type(4)));
  const u4v t = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// ---- cross-lane moves ------------------------------------------------------
// DPP controls (GCN/CDNA encoding): quad_perm selectors, row mirrors.
constexpr int DPP_QUAD_XOR1 = 0xB1;     // [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;     // [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }
__device__ __forceinline__ int shfl_xor_i(int v, int mask) { return __shfl_xor(v, mask, 64); }

// Max / sum over lane pairs (l, l ^ 16) and (l, l ^ 32) with gfx950's row
// swaps: a swap of (v, v) returns, in every lane, the two values of its pair
// (v_permlane16_swap exchanges odd and even 16-lane rows, v_permlane32_swap
// the wavefront halves), so a symmetric op of the two outputs is the pair's
// result in both lanes. One VALU op each, no LDS round trip.
// (v_max_f32 written directly: fmaxf would first quiet both inputs, two
// more ops, for signalling NaNs that the callers never produce)
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32_e32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum / max over aligned groups of LANES lanes (LANES in 1..64), result in
// every lane of the group. Groups of up to 16 lanes use DPP within a row.
template <int LANES>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LANES >= 2) v += dpp_f<DPP_QUAD_XOR1>(v);
  if constexpr (LANES >= 4) v += dpp_f<DPP_QUAD_XOR2>(v);
  if constexpr (LANES >= 8) v += dpp_f<DPP_ROW_HALF_MIRROR>(v);
  if constexpr (LANES >= 16) v += dpp_f<DPP_ROW_MIRROR>(v);
  if constexpr (LANES >= 32) v += shfl_xor_f(v, 16);
  if constexpr (LANES >= 64) v += shfl_xor_f(v, 32);
  return v;
}

template <int LANES>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (LANES >= 2) v = fmaxf(v, dpp_f<DPP_QUAD_XOR1>(v));
  if constexpr (LANES >= 4) v = fmaxf(v, dpp_f<DPP_QUAD_XOR2>(v));
  if constexpr (LANES >= 8) v = fmaxf(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
  if constexpr (LANES >= 16) v = fmaxf(v, dpp_f<DPP_ROW_MIRROR>(v));
  if constexpr (LANES >= 32) v = fmaxf(v, shfl_xor_f(v, 16));
  if constexpr (LANES >= 64) v = fmaxf(v, shfl_xor_f(v, 32));
  return v;
}

// Sum / max across lanes whose ids differ only in bits >= log2(FROM), i.e.
// over the 64/FROM groups of FROM lanes, for FROM in {1,..,64}.
template <int FROM>
__device__ __forceinline__ float across_groups_sum(float v) {
#pragma unroll
  for (int m = FROM; m < 64; m <<= 1) v += shfl_xor_f(v, m);
  return v;
}
template <int FROM>
__device__ __forceinline__ float across_groups_max(float v) {
#pragma unroll
  for (int m = FROM; m < 64; m <<= 1) v = fmaxf(v, shfl_xor_f(v, m));
  return v;
}

__device__ __forceinline__ void flag_error(uint32_t* err, uint32_t bit) {
  if (err) atomicOr(err, bit);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace zp
