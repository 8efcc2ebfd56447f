// Test probes (not part of libspecverify): the raw Philox4x64-10 words and uniforms the
// sampling kernels draw, written out so a test can compare them word for word with the
// oracle's generator, and the races' exponential variate -ln(1 - u).  They call the very
// device functions the sampling kernels use (sample_device.hpp), with their counter
// layout: key (seed, 0), counter (offset, b, (purpose << 32) | row, j >> 2), word j & 3.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sample_device.hpp"

namespace {

__global__ void philox_words_kernel(uint64_t seed, uint64_t offset, uint64_t b, uint64_t purpose,
                                    uint64_t row, uint64_t j0, int32_t n, uint64_t* words,
                                    double* unif) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint64_t j = j0 + static_cast<uint64_t>(i);
  const sv::U64x4 w = sv::philox(offset, b, (purpose << 32) | row, j >> 2, seed, 0);
  const uint64_t x = w.x[j & 3];
  words[i] = x;
  unif[i] = sv::to_uniform(x);
}

__global__ void neg_log1m_kernel(const double* u, double* e, int32_t n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) e[i] = sv::neg_log1m(u[i]);
}

}  // namespace

extern "C" {

// Writes words[i] and uniforms unif[i] of token ids j0 .. j0+n-1 (device arrays of n
// entries).  Returns 0, -1 for invalid arguments, or the HIP error of the launch.
int sv_probe_philox(uint64_t seed, uint64_t offset, uint64_t b, uint64_t purpose, uint64_t row,
                    uint64_t j0, int32_t n, void* words, void* unif, void* stream) {
  if (!words || !unif || n < 1 || purpose > 0xFFFFFFFFull || row > 0xFFFFFFFFull) return -1;
  hipLaunchKernelGGL(philox_words_kernel, dim3((n + 255) / 256), dim3(256), 0,
                     static_cast<hipStream_t>(stream), seed, offset, b, purpose, row, j0, n,
                     static_cast<uint64_t*>(words), static_cast<double*>(unif));
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : static_cast<int>(e);
}

// Writes e[i] = -ln(1 - u[i]) as the races compute it, for device arrays of n doubles
// (u in [0, 1)).  Returns 0, -1 for invalid arguments, or the HIP error of the launch.
int sv_probe_neg_log1m(const void* u, void* e, int32_t n, void* stream) {
  if (!u || !e || n < 1) return -1;
  hipLaunchKernelGGL(neg_log1m_kernel, dim3((n + 255) / 256), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const double*>(u),
                     static_cast<double*>(e), n);
  const hipError_t er = hipGetLastError();
  return er == hipSuccess ? 0 : static_cast<int>(er);
}

}  // extern "C"
