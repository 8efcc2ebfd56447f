// KV append: scatter n new token rows per sequence into the paged cache (token-major K
// pages, dim-major V pages).  Grid (token, KV head, sequence); one thread per element of
// the head_dim.
#include "common.hpp"
#include "internal.hpp"

namespace sv {
namespace {

// The fields the first loads need come first as plain arguments (preloaded into SGPRs).
template <typename E>
__global__ void __launch_bounds__(128)
kv_append_kernel(const int32_t* start, const int32_t* page_table, int32_t D, int32_t max_pages,
                 int32_t P_log2, int32_t num_pages, const AppendParams p) {
  const int e = threadIdx.x;
  const int t = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  if (e >= D) return;
  const int pos = start[b] + t;
  if (pos < 0 || pos >= (max_pages << P_log2)) return;
  const int page = page_table[static_cast<size_t>(b) * max_pages + (pos >> P_log2)];
  if (static_cast<unsigned>(page) >= static_cast<unsigned>(num_pages)) return;
  const int slot = pos & ((1 << P_log2) - 1);
  const size_t src = ((static_cast<size_t>(b) * p.n + t) * p.Hkv + g) * D + e;
  const size_t kdst = (((static_cast<size_t>(page) * p.Hkv + g) << P_log2) + slot) * D + e;
  const size_t vdst = (((static_cast<size_t>(page) * p.Hkv + g) * D + e) << P_log2) + slot;
  static_cast<E*>(p.k_cache)[kdst] = static_cast<const E*>(p.k_new)[src];
  static_cast<E*>(p.v_cache)[vdst] = static_cast<const E*>(p.v_new)[src];
}

}  // namespace

hipError_t launch_kv_append(const AppendParams& p, hipStream_t stream) {
  const dim3 grid(p.n, p.Hkv, p.B);
  if (p.elem_bytes == 2)
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, grid, dim3(128), 0, stream, p.start, p.page_table,
                       p.D, p.max_pages, p.P_log2, p.num_pages, p);
  else
    hipLaunchKernelGGL(kv_append_kernel<float>, grid, dim3(128), 0, stream, p.start, p.page_table,
                       p.D, p.max_pages, p.P_log2, p.num_pages, p);
  return hipGetLastError();
}

}  // namespace sv
