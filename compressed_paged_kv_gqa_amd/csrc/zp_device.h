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

// Raw buffer loads. A resource covers [base, base + bytes); a load whose
// offset falls outside it returns zeros and reads no memory, so an empty
// resource (bytes = 0) turns a load into a no-op that still counts as an
// outstanding load. Flags word: 32-bit data, no swizzle (the value CDNA
// buffer resources take).
typedef __amdgpu_buffer_rsrc_t BufRsrc;
__device__ __forceinline__ BufRsrc make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// 16 bytes at byte offset `off` of the resource, non-temporal (cache-policy
// bit 1).
__device__ __forceinline__ uint4 ldbuf16_nt(BufRsrc r, uint32_t off) {
  typedef unsigned int u4v __attribute__((ext_vector_type(4)));
  const u4v t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
  return make_uint4(t.x, t.y, t.z, t.w);
}

// ---- cross-lane moves ------------------------------------------------------
// DPP controls (GCN/CDNA encoding): quad_perm selectors, row mirrors.
constexpr int DPP_QUAD_XOR1 = 0xB1;     // [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;     // [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;
// Within each 16-lane row: lane i reads lane i + 4 (row_shl:4), lane i - 4
// (row_shr:4), lane (i + 8) mod 16 (row_ror:8, i.e. i ^ 8), and lane n of the
// row (row_newbcast:n, gfx90a and later). Sources outside the row give the
// `old` operand (0 in dpp_f) or 0 (dpp_z).
constexpr int DPP_ROW_SHL4 = 0x104;
constexpr int DPP_ROW_SHR4 = 0x114;
constexpr int DPP_ROW_ROR8 = 0x128;
constexpr int DPP_ROW_NEWBCAST0 = 0x150;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Same move with bound_ctrl set: lanes whose source is outside the row read
// 0 without a prior write of the destination.
template <int CTRL>
__device__ __forceinline__ float dpp_z(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }
__device__ __forceinline__ int shfl_xor_i(int v, int mask) { return __shfl_xor(v, mask, 64); }

// Max / sum over lane pairs (l, l ^ 16) and (l, l ^ 32) with gfx950's row
// swaps: a swap of (v, v) returns, in every lane, the two values of its pair
// (v_permlane16_swap exchanges odd and even 16-lane rows, v_permlane32_swap
// the wavefront halves), so a symmetric op of the two outputs is the pair's
// result in both lanes. One VALU op each, no LDS round trip.
// (fmaxf, not a hand-written v_max_f32: the compiler's hazard checks do not
// look inside inline asm, and a v_max_f32 issued right after a v_exp_f32 or
// a lane exchange that produced its operand can read the register's old
// value)
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lane n (0..15) of each 16-lane row, in every lane of the row; n must fold
// to a constant (unrolled loops), each case being one DPP move.
__device__ __forceinline__ float bcast_row_lane(float v, int n) {
  switch (n & 15) {
    case 0: return dpp_z<DPP_ROW_NEWBCAST0 + 0>(v);
    case 1: return dpp_z<DPP_ROW_NEWBCAST0 + 1>(v);
    case 2: return dpp_z<DPP_ROW_NEWBCAST0 + 2>(v);
    case 3: return dpp_z<DPP_ROW_NEWBCAST0 + 3>(v);
    case 4: return dpp_z<DPP_ROW_NEWBCAST0 + 4>(v);
    case 5: return dpp_z<DPP_ROW_NEWBCAST0 + 5>(v);
    case 6: return dpp_z<DPP_ROW_NEWBCAST0 + 6>(v);
    case 7: return dpp_z<DPP_ROW_NEWBCAST0 + 7>(v);
    case 8: return dpp_z<DPP_ROW_NEWBCAST0 + 8>(v);
    case 9: return dpp_z<DPP_ROW_NEWBCAST0 + 9>(v);
    case 10: return dpp_z<DPP_ROW_NEWBCAST0 + 10>(v);
    case 11: return dpp_z<DPP_ROW_NEWBCAST0 + 11>(v);
    case 12: return dpp_z<DPP_ROW_NEWBCAST0 + 12>(v);
    case 13: return dpp_z<DPP_ROW_NEWBCAST0 + 13>(v);
    case 14: return dpp_z<DPP_ROW_NEWBCAST0 + 14>(v);
    default: return dpp_z<DPP_ROW_NEWBCAST0 + 15>(v);
  }
}

// Transposing sum over each 16-lane row: x[i] (i = 0..15) are per-lane
// partial values; lane j of the row returns the row's total of x[j]. Each
// step halves the values a lane carries: at the step on lane bit k, a lane
// keeps the half whose index bit k equals its own bit k and sends the other
// half to its partner lane (bit k flipped), which keeps that half. 15 adds
// and ~36 selects/moves, against 64 adds for 16 separate all-reduces.
__device__ __forceinline__ float row_transpose_sum16(const float (&x)[16], int j) {
  const bool b0 = j & 1, b1 = j & 2, b2 = j & 4, b3 = j & 8;
  float w1[8], w2[4], w3[2];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float keep = b0 ? x[2 * k + 1] : x[2 * k], send = b0 ? x[2 * k] : x[2 * k + 1];
    w1[k] = keep + dpp_z<DPP_QUAD_XOR1>(send);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float keep = b1 ? w1[2 * k + 1] : w1[2 * k], send = b1 ? w1[2 * k] : w1[2 * k + 1];
    w2[k] = keep + dpp_z<DPP_QUAD_XOR2>(send);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float keep = b2 ? w2[2 * k + 1] : w2[2 * k], send = b2 ? w2[2 * k] : w2[2 * k + 1];
    const float up = dpp_z<DPP_ROW_SHL4>(send), dn = dpp_z<DPP_ROW_SHR4>(send);
    w3[k] = keep + (b2 ? dn : up);
  }
  const float keep = b3 ? w3[1] : w3[0], send = b3 ? w3[0] : w3[1];
  return keep + dpp_z<DPP_ROW_ROR8>(send);
}

// Sum / max over aligned groups of LANES lanes (LANES in 1..64), result in
// every lane of the group. Groups of up to 16 lanes use DPP within a row.
template <int LANES>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LANES >= 2) v += dpp_f<DPP_QUAD_XOR1>(v);
  if constexpr (LANES >= 4) v += dpp_f<DPP_QUAD_XOR2>(v);
  if constexpr (LANES >= 8) v += dpp_f<DPP_ROW_HALF_MIRROR>(v);
  if constexpr (LANES >= 16) v += dpp_f<DPP_ROW_MIRROR>(v);
  if constexpr (LANES >= 32) v = xor16_sum(v);
  if constexpr (LANES >= 64) v = xor32_sum(v);
  return v;
}

template <int LANES>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (LANES >= 2) v = fmaxf(v, dpp_f<DPP_QUAD_XOR1>(v));
  if constexpr (LANES >= 4) v = fmaxf(v, dpp_f<DPP_QUAD_XOR2>(v));
  if constexpr (LANES >= 8) v = fmaxf(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
  if constexpr (LANES >= 16) v = fmaxf(v, dpp_f<DPP_ROW_MIRROR>(v));
  if constexpr (LANES >= 32) v = xor16_max(v);
  if constexpr (LANES >= 64) v = xor32_max(v);
  return v;
}

// Sum / max across lanes whose ids differ only in bits >= log2(FROM), i.e.
// over the 64/FROM groups of FROM lanes, for FROM in {1,..,64}.
// The steps across 16-lane rows (lane ^ 16, lane ^ 32) take the row swaps
// above; the sums equal those of a shuffle bit for bit (a + b = b + a).
template <int FROM>
__device__ __forceinline__ float across_groups_sum(float v) {
#pragma unroll
  for (int m = FROM; m < 16; m <<= 1) v += shfl_xor_f(v, m);
  if constexpr (FROM <= 16) v = xor16_sum(v);
  if constexpr (FROM <= 32) v = xor32_sum(v);
  return v;
}
template <int FROM>
__device__ __forceinline__ float across_groups_max(float v) {
#pragma unroll
  for (int m = FROM; m < 16; m <<= 1) v = fmaxf(v, shfl_xor_f(v, m));
  if constexpr (FROM <= 16) v = xor16_max(v);
  if constexpr (FROM <= 32) v = xor32_max(v);
  return v;
}

__device__ __forceinline__ void flag_error(uint32_t* err, uint32_t bit) {
  if (err) atomicOr(err, bit);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace zp
