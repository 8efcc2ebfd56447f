// KV append: scatter n new token rows per sequence into the paged cache (token-major K
// pages, dim-major V pages).  Grid (token, KV head, sequence); one thread per element of
// the head_dim.
#include "common.hpp"
#include "internal.hpp"

namespace sv {
namespace {

template <typename E>
__global__ void __launch_bounds__(128) kv_append_kernel(const AppendParams p) {
  const int e = threadIdx.x;
  const int t = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  if (e >= p.D) return;
  const int pos = p.start[b] + t;
  if (pos < 0 || pos >= (p.max_pages << p.P_log2)) return;
  const int page = p.page_table[static_cast<size_t>(b) * p.max_pages + (pos >> p.P_log2)];
  if (static_cast<unsigned>(page) >= static_cast<unsigned>(p.num_pages)) return;
  const int slot = pos & ((1 << p.P_log2) - 1);
  const size_t src = ((static_cast<size_t>(b) * p.n + t) * p.Hkv + g) * p.D + e;
  const size_t kdst = (((static_cast<size_t>(page) * p.Hkv + g) << p.P_log2) + slot) * p.D + e;
  const size_t vdst = (((static_cast<size_t>(page) * p.Hkv + g) * p.D + e) << p.P_log2) + slot;
  static_cast<E*>(p.k_cache)[kdst] = static_cast<const E*>(p.k_new)[src];
  static_cast<E*>(p.v_cache)[vdst] = static_cast<const E*>(p.v_new)[src];
}

}  // namespace

hipError_t launch_kv_append(const AppendParams& p, hipStream_t stream) {
  const dim3 grid(p.n, p.Hkv, p.B);
  if (p.elem_bytes == 2)
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, grid, dim3(128), 0, stream, p);
  else
    hipLaunchKernelGGL(kv_append_kernel<float>, grid, dim3(128), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sv
