// Device helpers shared by the HIP kernels of libqas (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qas {

constexpr int kWave = 64;

// Storage dtypes (values of qas_dtype).
enum : int { kF32 = 0, kF16 = 1, kBF16 = 2, kE4M3 = 3 };

template <int DT> struct DType;
template <> struct DType<kF32> { static constexpr int bytes = 4; };
template <> struct DType<kF16> { static constexpr int bytes = 2; };
template <> struct DType<kBF16> { static constexpr int bytes = 2; };
template <> struct DType<kE4M3> { static constexpr int bytes = 1; };

// Elements held by one 16-byte load.
template <int DT> constexpr int epl() { return 16 / DType<DT>::bytes; }

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// Decode one 16-byte chunk into epl<DT>() floats (exact for every format).
template <int DT>
__device__ __forceinline__ void unpack16(const uint4& raw, float* out);

template <>
__device__ __forceinline__ void unpack16<kF32>(const uint4& raw, float* out) {
  out[0] = __uint_as_float(raw.x);
  out[1] = __uint_as_float(raw.y);
  out[2] = __uint_as_float(raw.z);
  out[3] = __uint_as_float(raw.w);
}

template <>
__device__ __forceinline__ void unpack16<kF16>(const uint4& raw, float* out) {
  half8_t h = __builtin_bit_cast(half8_t, raw);
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = (float)h[i];
}

template <>
__device__ __forceinline__ void unpack16<kBF16>(const uint4& raw, float* out) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Convert a float that is exactly representable in DT back to storage bits
// (used for min/max summaries, whose values are always input values).
template <int DT> struct Store;
template <> struct Store<kF32> {
  typedef float T;
  static __device__ __forceinline__ T from(float v) { return v; }
};
template <> struct Store<kF16> {
  typedef _Float16 T;
  static __device__ __forceinline__ T from(float v) { return (_Float16)v; }
};
template <> struct Store<kBF16> {
  typedef uint16_t T;
  static __device__ __forceinline__ T from(float v) {
    return (uint16_t)(__float_as_uint(v) >> 16);
  }
};

// Round-to-nearest-even float -> storage (outputs).
template <int DT> __device__ __forceinline__ void store_rn(void* base, size_t i, float v);
template <> __device__ __forceinline__ void store_rn<kF32>(void* base, size_t i, float v) {
  reinterpret_cast<float*>(base)[i] = v;
}
template <> __device__ __forceinline__ void store_rn<kF16>(void* base, size_t i, float v) {
  reinterpret_cast<_Float16*>(base)[i] = (_Float16)v;
}
template <> __device__ __forceinline__ void store_rn<kBF16>(void* base, size_t i, float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7f800000u) == 0x7f800000u) {          // inf / nan: keep, quiet nan
    u = (u & 0x007fffffu) ? (u | 0x00400000u) : u;
  } else {
    u += 0x7fffu + ((u >> 16) & 1u);               // nearest, ties to even
  }
  reinterpret_cast<uint16_t*>(base)[i] = (uint16_t)(u >> 16);
}

template <int DT> __device__ __forceinline__ float load_scalar(const void* base, size_t i);
template <> __device__ __forceinline__ float load_scalar<kF32>(const void* base, size_t i) {
  return reinterpret_cast<const float*>(base)[i];
}
template <> __device__ __forceinline__ float load_scalar<kF16>(const void* base, size_t i) {
  return (float)reinterpret_cast<const _Float16*>(base)[i];
}
template <> __device__ __forceinline__ float load_scalar<kBF16>(const void* base, size_t i) {
  return __uint_as_float(((uint32_t)reinterpret_cast<const uint16_t*>(base)[i]) << 16);
}

__device__ __forceinline__ uint4 load16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// ---- cross-lane reductions over aligned lane groups -----------------------
// Inside a 16-lane row these use DPP (GFX9 encoding): quad_perm [1,0,3,2]
// (0xB1) and [2,3,0,1] (0x4E) leave every lane of a quad with the quad's
// value; row_half_mirror (0x141, lane i <- 7-i of its half-row) then joins
// the two quads of each half-row, and row_mirror (0x140, lane i <- 15-i)
// joins the two half-rows.  Groups of 32 and 64 lanes add xor shuffles.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N lanes (N a power of two <= 64); every lane of the
// group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_f<0xB1>(v);
  if constexpr (N >= 4) v += dpp_f<0x4E>(v);
  if constexpr (N >= 8) v += dpp_f<0x141>(v);
  if constexpr (N >= 16) v += dpp_f<0x140>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16, kWave);
  if constexpr (N >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

template <int N>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (N >= 2) v = fmaxf(v, dpp_f<0xB1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp_f<0x4E>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp_f<0x141>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp_f<0x140>(v));
  if constexpr (N >= 32) v = fmaxf(v, __shfl_xor(v, 16, kWave));
  if constexpr (N >= 64) v = fmaxf(v, __shfl_xor(v, 32, kWave));
  return v;
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

// exp2 with exp2(-inf) = 0, via the hardware v_exp_f32.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Order-preserving map float -> uint32 (larger float -> larger key); -0 and
// +0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---- e4m3 (OCP fn) codes with a chosen rounding direction ----------------
// Codes are sign-magnitude: for a non-negative code one step up in value is
// code + 1; for a negative code (bit 7) it is code - 1.  -0 (0x80) and +0
// both mean zero.

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  return __builtin_amdgcn_cvt_f32_fp8((int)c, 0);
}

// nearest-even code of x, |x| <= 448 (the conversion would not saturate)
__device__ __forceinline__ uint32_t e4m3_nearest(float x) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false) & 0xffu;
}

// largest e4m3 value <= x and smallest e4m3 value >= x, for |x| <= 448
__device__ __forceinline__ uint32_t e4m3_down(float x) {
  uint32_t c = e4m3_nearest(x);
  if (e4m3_value(c) > x) c = (c & 0x80u) ? c + 1u : (c == 0u ? 0x81u : c - 1u);
  return c;
}
__device__ __forceinline__ uint32_t e4m3_up(float x) {
  uint32_t c = e4m3_nearest(x);
  if (e4m3_value(c) < x) c = (c & 0x80u) ? (c == 0x80u ? 0x01u : c - 1u) : c + 1u;
  return c;
}

// Smallest k with amax <= 448 * 2^k (0 for amax = 0): with amax = f * 2^e,
// f in [0.5, 1), 448 = 0.875 * 2^9 gives k = e - 9, or e - 8 if f > 0.875.
__device__ __forceinline__ int summary_scale_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int e;
  const float f = frexpf(amax, &e);
  return e - 9 + (f > 0.875f ? 1 : 0);
}

}  // namespace qas
