// Shared device-side helpers for the gfx950 kernels: bf16 conversion, MFMA operand types,
// wave reductions. Device code only; no host logic lives here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace q3 {

__device__ __forceinline__ float bf2f(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Load element i of a weight vector stored as bf16 (is_bf16) or f32.
__device__ __forceinline__ float load_w(const void* w, int i, bool is_bf16) {
  return is_bf16 ? bf2f(static_cast<const uint16_t*>(w)[i]) : static_cast<const float*>(w)[i];
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int o = width >> 1; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-bit matrix-product operand formats.
enum Op16 : int { OP_BF16 = 0, OP_F16 = 1 };

__device__ __forceinline__ float h2f(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}
__device__ __forceinline__ uint16_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// Per-format helpers: 32x32x16 MFMA on 8-element operands held as u32x4, conversions.
template <int OP>
struct Fmt;

template <>
struct Fmt<OP_BF16> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ float to_f32(uint16_t h) { return bf2f(h); }
  static __device__ __forceinline__ uint16_t from_f32(float f) { return f2bf(f); }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) { return pack2bf(lo, hi); }
  // acc + lo + hi of a packed pair (one v_dot2 against (1, 1), fp32 accumulation)
  static __device__ __forceinline__ float sum2(uint32_t w, float acc) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                           __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc, false);
  }
};

template <>
struct Fmt<OP_F16> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ float to_f32(uint16_t h) { return h2f(h); }
  static __device__ __forceinline__ uint16_t from_f32(float f) { return f2h(f); }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2 v = {lo, hi};
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
  }
  // acc + lo + hi of a packed pair (one v_dot2 against (1, 1), fp32 accumulation)
  static __device__ __forceinline__ float sum2(uint32_t w, float acc) {
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w), __builtin_bit_cast(f16x2_t, 0x3c003c00u), acc,
                                  false);
  }
};

// Two bf16 values (one 32-bit word) -> two fp16 values. A bf16 value converts exactly when
// its magnitude lies in [2^-17, 65504]; smaller magnitudes truncate toward zero with an
// absolute error below 2^-24.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  const float lo = __uint_as_float(w << 16);
  const float hi = __uint_as_float(w & 0xFFFF0000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// 8 consecutive elements starting at src + i (element index), as floats; one 16-byte load for
// 16-bit types, two for fp32. DT is a DType.
template <int DT>
__device__ __forceinline__ void load8(const void* src, int64_t i, float (&v)[8]) {
  if (DT == DT_F32) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(src) + i);
    const f32x4 b = *reinterpret_cast<const f32x4*>(static_cast<const float*>(src) + i + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  } else {
    const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t lo = static_cast<uint16_t>(w[e] & 0xFFFF), hi = static_cast<uint16_t>(w[e] >> 16);
      v[2 * e] = DT == DT_BF16 ? bf2f(lo) : h2f(lo);
      v[2 * e + 1] = DT == DT_BF16 ? bf2f(hi) : h2f(hi);
    }
  }
}

// The inverse of load8: 8 floats stored at dst + i, rounded to nearest even for 16-bit types.
template <int DT>
__device__ __forceinline__ void store8(void* dst, int64_t i, const float (&v)[8]) {
  if (DT == DT_F32) {
    float* d = static_cast<float*>(dst) + i;
    *reinterpret_cast<f32x4*>(d) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(d + 4) = f32x4{v[4], v[5], v[6], v[7]};
  } else {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = DT == DT_BF16 ? Fmt<OP_BF16>::pack2(v[2 * e], v[2 * e + 1]) : Fmt<OP_F16>::pack2(v[2 * e], v[2 * e + 1]);
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(dst) + i) = w;
  }
}

}  // namespace q3
