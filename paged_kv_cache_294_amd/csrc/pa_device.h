// Device helpers shared by the paged-attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kBlockSize = 16;  // tokens per KV block

// Pool element offset of (slot, kv) row start: pool is [NB][16][2][Hkv][D].
__device__ __forceinline__ int64_t row_offset(int64_t slot, int kv, int kv_row_elems) {
  return (slot * 2 + kv) * (int64_t)kv_row_elems;
}

// DPP lane moves (gfx9 encodings). Only row-local patterns are used.
enum : int {
  kDppXor1 = 0xB1,         // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,         // quad_perm [2,3,0,1]
  kDppHalfMirror = 0x141,  // lane i <-> 7-i inside each half row of 8
  kDppMirror = 0x140,      // lane i <-> 15-i inside each row of 16
};

template <int Ctrl>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), Ctrl, 0xF, 0xF, false));
}

// Sum over groups of N consecutive lanes (N in {4, 8, 16}) aligned to N; every lane of the
// group gets the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16, "row-local sums only");
  x += dpp_mov<kDppXor1>(x);
  x += dpp_mov<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp_mov<kDppHalfMirror>(x);
  if constexpr (N == 16) x += dpp_mov<kDppMirror>(x);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte load from global memory. The explicit global address space keeps the compiler
// from falling back to flat loads (which also count against the LDS wait counter) when
// it cannot trace a pointer back to a kernel argument. With Stream the load carries the
// non-temporal hint, for data read once.
typedef __attribute__((address_space(1))) const half8_t gconst_half8_t;

template <bool Stream = false>
__device__ __forceinline__ half8_t load16(const half_t* p) {
  gconst_half8_t* gp = (gconst_half8_t*)(p);
  if constexpr (Stream)
    return __builtin_nontemporal_load(gp);
  else
    return *gp;
}

// FP8 (OCP E4M3) cache elements are stored as bytes.
typedef uint8_t fp8_t;
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const u32x2_t gconst_u32x2_t;

// Eight E4M3 codes (in memory order) widened exactly to fp16: every E4M3 value is an fp16
// value, and v_cvt_scalef32_pk_f16_fp8 with scale 1 converts two codes.
__device__ __forceinline__ half8_t widen_fp8x8(u32x2_t w) {
  const half2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.0f, false);
  const half2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.0f, true);
  const half2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.0f, false);
  const half2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.0f, true);
  return half8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Eight consecutive cache elements as fp16: a 16-byte load of fp16 elements, or an 8-byte
// load of E4M3 codes widened to fp16.
template <typename KV, bool Stream = false>
__device__ __forceinline__ half8_t load_kv8(const KV* p) {
  if constexpr (sizeof(KV) == 2) {
    return load16<Stream>(reinterpret_cast<const half_t*>(p));
  } else {
    gconst_u32x2_t* gp = (gconst_u32x2_t*)(p);
    u32x2_t w;
    if constexpr (Stream)
      w = __builtin_nontemporal_load(gp);
    else
      w = *gp;
    return widen_fp8x8(w);
  }
}

// E4M3 code of a NaN: the NaN pattern with the input's sign.
__device__ __forceinline__ unsigned int fp8_nan(float x) {
  return 0x7Fu | ((__builtin_bit_cast(unsigned int, x) >> 24) & 0x80u);
}

// Two fp32 values as E4M3 codes in the low 16 bits, round to nearest even. The hardware
// conversion turns magnitudes past the 448 / 480 midpoint into NaN, so values are first
// clamped to +-448 (saturation); it also gives every NaN the negative NaN code, so NaN
// inputs get their sign back.
__device__ __forceinline__ unsigned int fp8x2(float x, float y) {
  const unsigned int c = (unsigned int)__builtin_amdgcn_cvt_pk_fp8_f32(
      fminf(fmaxf(x, -448.0f), 448.0f), fminf(fmaxf(y, -448.0f), 448.0f), 0, false);
  const unsigned int lo = (x != x) ? fp8_nan(x) : (c & 0xFFu);
  const unsigned int hi = (y != y) ? fp8_nan(y) : ((c >> 8) & 0xFFu);
  return lo | (hi << 8);
}

__device__ __forceinline__ float dot8(half8_t a, half8_t b, float acc) {
  acc = __builtin_amdgcn_fdot2(half2_t{a[0], a[1]}, half2_t{b[0], b[1]}, acc, false);
  acc = __builtin_amdgcn_fdot2(half2_t{a[2], a[3]}, half2_t{b[2], b[3]}, acc, false);
  acc = __builtin_amdgcn_fdot2(half2_t{a[4], a[5]}, half2_t{b[4], b[5]}, acc, false);
  acc = __builtin_amdgcn_fdot2(half2_t{a[6], a[7]}, half2_t{b[6], b[7]}, acc, false);
  return acc;
}

// Max and sum of x over lanes L and L ^ O of a wave. For O = 16 and 32 gfx950's
// v_permlane16_swap / v_permlane32_swap exchange rows of 16 lanes (halves of 32 lanes)
// between two registers inside the vector ALU, without the LDS round trip of ds_bpermute:
// with x in both operands, the two results hold x of the lane and x of its partner, in an
// order that depends on the lane, which max and sum do not see (both are commutative, so
// every lane of a pair gets the same bits as with a shuffle).
template <int O>
__device__ __forceinline__ float max_xor(float x) {
  if constexpr (O == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else if constexpr (O == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else {
    return fmaxf(x, __shfl_xor(x, O, kWave));
  }
}

template <int O>
__device__ __forceinline__ float sum_xor(float x) {
  if constexpr (O == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else if constexpr (O == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    return x + __shfl_xor(x, O, kWave);
  }
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }
__device__ __forceinline__ float qnan() { return __builtin_nanf(""); }

}  // namespace pkv
