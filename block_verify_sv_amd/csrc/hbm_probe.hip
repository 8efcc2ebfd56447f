// Streaming-read probe for the HBM roofline (measurement only; not part of
// libspecverify).  It answers one question: how fast can a plain, hand-written kernel
// read a given number of bytes from HBM on this GPU, as one launch?  The verify-attention
// pass reads its KV cache exactly once, so this is the ceiling its bandwidth is measured
// against next to the 8 TB/s data-sheet peak.
//
// Each thread issues `kLoads` 16-byte loads per round, all in flight before any is
// consumed; consecutive lanes read consecutive 16-byte words (fully coalesced 1 KB per
// wave per load).  Workgroups take contiguous stretches of the buffer, in rounds of
// `kLoads * kThreads * 16` bytes, so each stretch is a run of whole DRAM pages.  The
// loaded words are folded into an XOR that is written only if it equals a value the
// data never produces, which keeps every load alive without adding write traffic.
// The loads are either ordinary or non-temporal (streaming); the faster of the two is
// the ceiling.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kLoads = 8;
constexpr uint32_t kNever = 0x9E3779B9u;

template <bool NT>
__global__ void __launch_bounds__(kThreads)
hbm_read_kernel(const u32x4* src, uint64_t n16, uint64_t per_wg, u32x4* sink) {
  const uint64_t begin = static_cast<uint64_t>(blockIdx.x) * per_wg;
  uint64_t end = begin + per_wg;
  if (end > n16) end = n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  constexpr uint64_t kRound = static_cast<uint64_t>(kLoads) * kThreads;
  for (uint64_t r = begin; r < end; r += kRound) {
    u32x4 v[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const uint64_t i = r + static_cast<uint64_t>(u) * kThreads + threadIdx.x;
      const u32x4* a = src + (i < end ? i : end - 1);  // clamped: in bounds, counted once below
      if constexpr (NT)
        v[u] = __builtin_nontemporal_load(a);
      else
        v[u] = *a;
    }
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const uint64_t i = r + static_cast<uint64_t>(u) * kThreads + threadIdx.x;
      if (i < end) acc ^= v[u];
    }
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == kNever) sink[blockIdx.x * kThreads + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// Workgroups the probe launches for `bytes` at `wg_bytes` bytes per workgroup.
uint64_t sv_probe_workgroups(uint64_t bytes, uint64_t wg_bytes) {
  if (wg_bytes < 16) wg_bytes = 16;
  return (bytes + wg_bytes - 1) / wg_bytes;
}

// Reads `bytes` (a multiple of 16) at `src` (16-byte aligned) once, in one launch of
// ceil(bytes / wg_bytes) workgroups of 256 threads.  `sink` must hold
// 16 * 256 * sv_probe_workgroups(bytes, wg_bytes) bytes; it is written only in the
// (never occurring) case described above.  nontemporal != 0 reads with non-temporal
// loads.  Returns 0, or -1 for invalid arguments, or the HIP error code of the launch.
int sv_probe_read(const void* src, uint64_t bytes, uint64_t wg_bytes, int nontemporal,
                  void* sink, void* stream) {
  if (!src || !sink || bytes == 0 || (bytes & 15u) || (reinterpret_cast<uintptr_t>(src) & 15u))
    return -1;
  if (wg_bytes < 16 || (wg_bytes & 15u)) return -1;
  const uint64_t grid = sv_probe_workgroups(bytes, wg_bytes);
  if (grid > 0x7FFFFFFFull) return -1;
  if (nontemporal)
    hipLaunchKernelGGL(hbm_read_kernel<true>, dim3(static_cast<unsigned>(grid)), dim3(kThreads),
                       0, static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                       bytes / 16, wg_bytes / 16, static_cast<u32x4*>(sink));
  else
    hipLaunchKernelGGL(hbm_read_kernel<false>, dim3(static_cast<unsigned>(grid)), dim3(kThreads),
                       0, static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                       bytes / 16, wg_bytes / 16, static_cast<u32x4*>(sink));
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : static_cast<int>(e);
}

}  // extern "C"
