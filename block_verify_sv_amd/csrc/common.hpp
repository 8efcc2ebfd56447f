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
// Cross-lane exchange without an LDS round trip.  Stage S (0..5) pairs every lane with a
// lane in the other half of its aligned group of 2^(S+1) lanes: lane ^ 1 and lane ^ 2 (DPP
// quad permutes), the mirror lane within 8 and within 16 (DPP row half-mirror and row
// mirror), then lane ^ 16 and lane ^ 32 (the gfx950 row and half swaps).  After stages
// 0 .. S-1 of a reduction every lane of an aligned group of 2^S lanes holds the same
// value, so each stage combines two complete halves; the combining operations used here
// are commutative, so every lane of the group ends with bitwise the same result.
template <int S>
__device__ __forceinline__ uint32_t xlane(uint32_t v) {
  static_assert(S >= 0 && S < 6, "stage");
  if constexpr (S == 0) return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false));
  else if constexpr (S == 1) return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false));
  else if constexpr (S == 2) return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x141, 0xF, 0xF, false));
  else if constexpr (S == 3) return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x140, 0xF, 0xF, false));
  else if constexpr (S == 4) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
}
template <int S>
__device__ __forceinline__ uint64_t xlane64(uint64_t v) {
  const uint32_t lo = xlane<S>(static_cast<uint32_t>(v));
  const uint32_t hi = xlane<S>(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
template <int S>
__device__ __forceinline__ float xlane_f32(float v) { return __uint_as_float(xlane<S>(__float_as_uint(v))); }
template <int S>
__device__ __forceinline__ double xlane_f64(double v) {
  return __builtin_bit_cast(double, xlane64<S>(__builtin_bit_cast(uint64_t, v)));
}

// Reductions over aligned groups of 2^N lanes (N = 6: the whole wave).
template <int N = 6>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (N > 0) v = fmaxf(v, xlane_f32<0>(v));
  if constexpr (N > 1) v = fmaxf(v, xlane_f32<1>(v));
  if constexpr (N > 2) v = fmaxf(v, xlane_f32<2>(v));
  if constexpr (N > 3) v = fmaxf(v, xlane_f32<3>(v));
  if constexpr (N > 4) v = fmaxf(v, xlane_f32<4>(v));
  if constexpr (N > 5) v = fmaxf(v, xlane_f32<5>(v));
  return v;
}
template <int N = 6>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N > 0) v += xlane_f32<0>(v);
  if constexpr (N > 1) v += xlane_f32<1>(v);
  if constexpr (N > 2) v += xlane_f32<2>(v);
  if constexpr (N > 3) v += xlane_f32<3>(v);
  if constexpr (N > 4) v += xlane_f32<4>(v);
  if constexpr (N > 5) v += xlane_f32<5>(v);
  return v;
}
template <int N = 6>
__device__ __forceinline__ double group_sum_f64(double v) {
  if constexpr (N > 0) v += xlane_f64<0>(v);
  if constexpr (N > 1) v += xlane_f64<1>(v);
  if constexpr (N > 2) v += xlane_f64<2>(v);
  if constexpr (N > 3) v += xlane_f64<3>(v);
  if constexpr (N > 4) v += xlane_f64<4>(v);
  if constexpr (N > 5) v += xlane_f64<5>(v);
  return v;
}
template <int N = 6>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
  uint64_t w;
  if constexpr (N > 0) { w = xlane64<0>(v); v = w > v ? w : v; }
  if constexpr (N > 1) { w = xlane64<1>(v); v = w > v ? w : v; }
  if constexpr (N > 2) { w = xlane64<2>(v); v = w > v ? w : v; }
  if constexpr (N > 3) { w = xlane64<3>(v); v = w > v ? w : v; }
  if constexpr (N > 4) { w = xlane64<4>(v); v = w > v ? w : v; }
  if constexpr (N > 5) { w = xlane64<5>(v); v = w > v ? w : v; }
  return v;
}

__device__ __forceinline__ float wave_max(float v) { return group_max<6>(v); }
__device__ __forceinline__ double wave_sum_f64(double v) { return group_sum_f64<6>(v); }
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) { return group_max_u64<6>(v); }

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
