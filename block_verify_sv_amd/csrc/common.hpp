// Device helpers shared by the libspecverify kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ------------------------------------------------------------------ scalar conversions

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Conversions below use the gfx950 packed converts (v_cvt_pk_bf16_f32 /
// v_cvt_pk_f16_f32), which round to nearest even in the default rounding mode.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// Packs two floats into one dword of 16-bit values (lo first).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  const f16x2 v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// 2^x on the hardware exp unit (v_exp_f32): results below the normal range flush to 0,
// which is what a softmax weight that small should be.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------------ element tags
// KPL = elements of the contraction dimension one lane holds per MFMA operand
// (32x32x16 for 16-bit types, 32x32x2 for fp32).

struct TagBF16 {
  using store_t = uint16_t;
  static constexpr int kBytes = 2;
  static constexpr int KPL = 8;
  __device__ static float to_f32(store_t x) { return bf16_to_f32(x); }
  __device__ static store_t from_f32(float x) { return f32_to_bf16(x); }
  __device__ static uint32_t pack2(float a, float b) { return pack_bf16(a, b); }
};

struct TagF16 {
  using store_t = uint16_t;
  static constexpr int kBytes = 2;
  static constexpr int KPL = 8;
  __device__ static float to_f32(store_t x) { return f16_to_f32(x); }
  __device__ static store_t from_f32(float x) { return f32_to_f16(x); }
  __device__ static uint32_t pack2(float a, float b) { return pack_f16(a, b); }
};

struct TagF32 {
  using store_t = float;
  static constexpr int kBytes = 4;
  static constexpr int KPL = 1;
  __device__ static float to_f32(store_t x) { return x; }
  __device__ static store_t from_f32(float x) { return x; }
};

// One MFMA step on operands held as raw dwords: 4 dwords (8 x 16-bit) or 1 dword (fp32).
template <class Tag>
struct Mfma;

template <>
struct Mfma<TagBF16> {
  using op_t = u32x4;
  __device__ static f32x16 step(op_t a, op_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <>
struct Mfma<TagF16> {
  using op_t = u32x4;
  __device__ static f32x16 step(op_t a, op_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

template <>
struct Mfma<TagF32> {
  using op_t = float;
  __device__ static f32x16 step(op_t a, op_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// ------------------------------------------------------------------ wave reductions

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o);
    v = w > v ? w : v;
  }
  return v;
}

// Order-preserving map of a finite float to uint32 (-0.0 is folded onto +0.0, so equal
// values give equal keys).
__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 64-bit argmax key: larger value first, then the lower index.
__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t idx) {
  return (static_cast<uint64_t>(orderable(v)) << 32) | static_cast<uint64_t>(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ uint32_t argmax_key_index(uint64_t key) {
  return 0xFFFFFFFFu - static_cast<uint32_t>(key & 0xFFFFFFFFull);
}

}  // namespace sv
