// Device helpers shared by the sampling-acceptance kernels (chain and tree): the
// Philox4x64-10 generator and its uniforms, logit access, and the (key, index) minimum of
// the exponential race.
#pragma once

#include <math.h>
#include <stdint.h>

#include "common.hpp"

namespace sv {
namespace {

// An unwritten partial-result slot that a later workgroup of the same launch waits on:
// a signalling NaN, which no floating-point operation returns.  Producers publish with
// agent-scope atomic stores, consumers poll with agent-scope atomic loads, at most the
// call's wait limit of times (a kernel argument, sv_set_wait_limit), so every wave ends
// whatever happens.
constexpr uint64_t kSlotEmpty = 0x7FF5A5A5A5A5A5A5ull;
constexpr int32_t kIdxEmpty = -1;                 // an unwritten race index slot
constexpr int32_t kGaveUp = -2;                   // a race key entered for a wait that gave up

// ---- Philox4x64-10 (Salmon et al., SC'11): multipliers and Weyl key increments of
// the 4x64 variant; ten rounds.
constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kPhiloxW1 = 0xBB67AE8584CAA73Bull;

struct U64x4 {
  uint64_t x[4];
};

__device__ __forceinline__ U64x4 philox(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                        uint64_t k0, uint64_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    const uint64_t hi0 = __umul64hi(kPhiloxM0, c0), lo0 = kPhiloxM0 * c0;
    const uint64_t hi1 = __umul64hi(kPhiloxM1, c2), lo1 = kPhiloxM1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return U64x4{{c0, c1, c2, c3}};
}

__device__ __forceinline__ double to_uniform(uint64_t w) {
  return static_cast<double>(w >> 11) * 0x1.0p-53;
}

// E = -ln(1 - u) for a uniform u in [0, 1) on the 2^-53 grid, in fp64: the exponential
// variate of the race.  1 - u is exact; with 1 - u = m 2^k, m in [sqrt(1/2), sqrt(2)),
// ln m = 2 atanh(s), s = (m - 1) / (m + 1), |s| <= 0.172, summed as the odd series
// 2 (s + s^3/3 + ... + s^21/21) (truncation below 2^-60 relative), and k ln 2 with ln 2
// split in two parts.  About 35 instructions against 136 for the library log1p; the
// result is within a few ulp of -log1p(-u).
__device__ __forceinline__ double neg_log1m(double u) {
  // ln 2 in two parts: hi is ln 2 rounded to a multiple of 2^-32 (so k * hi is exact for
  // |k| < 2^20), lo = ln 2 - hi rounded to fp64
  constexpr double kLn2Hi = 0x1.62e42ff000000p-1;
  constexpr double kLn2Lo = -0x1.718432a1b0e26p-35;
  const double x = 1.0 - u;
  int k;
  double m = frexp(x, &k);                         // x = m 2^k, m in [1/2, 1)
  if (m < 0.70710678118654752440) {
    m *= 2.0;
    --k;
  }
  const double s = (m - 1.0) / (m + 1.0);
  const double z = s * s;
  double q = 1.0 / 21.0;
  q = fma(q, z, 1.0 / 19.0);
  q = fma(q, z, 1.0 / 17.0);
  q = fma(q, z, 1.0 / 15.0);
  q = fma(q, z, 1.0 / 13.0);
  q = fma(q, z, 1.0 / 11.0);
  q = fma(q, z, 1.0 / 9.0);
  q = fma(q, z, 1.0 / 7.0);
  q = fma(q, z, 1.0 / 5.0);
  q = fma(q, z, 1.0 / 3.0);
  const double lm = 2.0 * fma(s * z, q, s);        // ln m
  const double dk = static_cast<double>(k);
  return -(fma(dk, kLn2Hi, fma(dk, kLn2Lo, lm)));
}

template <bool kBF16>
__device__ __forceinline__ float logit_at(const void* base, size_t i) {
  if constexpr (kBF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
  else return static_cast<const float*>(base)[i];
}

__device__ __forceinline__ bool better(double k, int32_t i, double bk, int32_t bi) {
  return k < bk || (k == bk && i < bi);
}

// Smallest (key, index) of a workgroup, for the residual race and the p race.
// One exchange stage of the (key, index) minimum of two races (better() is symmetric).
template <int S>
__device__ __forceinline__ void best_stage(double& bk_r, int32_t& bi_r, double& bk_p, int32_t& bi_p) {
  const double kr = xlane_f64<S>(bk_r);
  const int32_t ir = static_cast<int32_t>(xlane<S>(static_cast<uint32_t>(bi_r)));
  if (better(kr, ir, bk_r, bi_r)) { bk_r = kr; bi_r = ir; }
  const double kp = xlane_f64<S>(bk_p);
  const int32_t ip = static_cast<int32_t>(xlane<S>(static_cast<uint32_t>(bi_p)));
  if (better(kp, ip, bk_p, bi_p)) { bk_p = kp; bi_p = ip; }
}

template <int kThreads>
__device__ __forceinline__ void block_best(double& bk_r, int32_t& bi_r, double& bk_p,
                                           int32_t& bi_p, double (*rk)[kThreads / kWave],
                                           int32_t (*ri)[kThreads / kWave]) {
  const int tid = threadIdx.x;
  best_stage<0>(bk_r, bi_r, bk_p, bi_p);
  best_stage<1>(bk_r, bi_r, bk_p, bi_p);
  best_stage<2>(bk_r, bi_r, bk_p, bi_p);
  best_stage<3>(bk_r, bi_r, bk_p, bi_p);
  best_stage<4>(bk_r, bi_r, bk_p, bi_p);
  best_stage<5>(bk_r, bi_r, bk_p, bi_p);
  if ((tid & 63) == 0) {
    rk[0][tid >> 6] = bk_r;
    ri[0][tid >> 6] = bi_r;
    rk[1][tid >> 6] = bk_p;
    ri[1][tid >> 6] = bi_p;
  }
  __syncthreads();
  bk_r = rk[0][0]; bi_r = ri[0][0]; bk_p = rk[1][0]; bi_p = ri[1][0];
#pragma unroll
  for (int w = 1; w < kThreads / kWave; ++w) {
    if (better(rk[0][w], ri[0][w], bk_r, bi_r)) { bk_r = rk[0][w]; bi_r = ri[0][w]; }
    if (better(rk[1][w], ri[1][w], bk_p, bi_p)) { bk_p = rk[1][w]; bi_p = ri[1][w]; }
  }
}

}  // namespace
}  // namespace sv
