// Cycle commit: after acceptance, the context of every sequence grows by the anchor plus
// its accepted drafts, whose K/V rows were written before the verify pass, and the
// target's token at the first disagreement becomes the next anchor (VFlash-FM page,
// caption of the cycle figure).  Rejected drafts' rows need no undo: the next block's
// append overwrites them.  One thread per sequence; the state never leaves the device.
#include "common.hpp"
#include "internal.hpp"

namespace sv {
namespace {

constexpr int kThreads = 256;

// Both kernels take the fields their first loads need as leading plain arguments
// (preloaded into SGPRs), then the whole parameter block.
__global__ void __launch_bounds__(kThreads)
commit_kernel(const int32_t* accept_len, const int32_t* out_tokens, int32_t B, int32_t K,
              const CommitParams p) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= B) return;
  int a = accept_len[b];
  a = a < 0 ? 0 : (a > K - 1 ? K - 1 : a);
  p.next_anchor[b] = out_tokens[static_cast<size_t>(b) * K + a];
  p.ctx_lens[b] += a + 1;
}

// Tree commit, before the commit above: the block was appended in node order at
// ctx .. ctx+K-1, and the accepted path's rows move to ctx+1 .. ctx+a (the j-th path node
// from ctx + path[j] to ctx + j; the anchor stays).  One workgroup per (KV head,
// sequence), one thread per element of a K row and of a V column.  Every source row is
// read (into LDS) before any destination is written, so a destination that is also a
// later node's source is never overwritten early.  Positions outside the page table and
// table entries outside the pool are skipped.
template <typename T>
__global__ void __launch_bounds__(128)
tree_compact_kernel(const int32_t* accept_len, const int32_t* ctx_lens,
                    const int32_t* page_table, const int32_t* paths, int32_t K, int32_t D,
                    int32_t max_pages, int32_t P_log2, const TreeCompactParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  T* const ks = reinterpret_cast<T*>(smem);      // [K-1][D]
  T* const vs = ks + static_cast<size_t>(K - 1) * D;
  const int g = blockIdx.x, b = blockIdx.y, x = threadIdx.x;
  if (x >= D) return;
  int a = accept_len[b];
  a = a < 0 ? 0 : (a > K - 1 ? K - 1 : a);
  const int ctx = ctx_lens[b];
  if (ctx < 0 || static_cast<int64_t>(ctx) + K > (static_cast<int64_t>(max_pages) << P_log2))
    return;
  const int Pm1 = (1 << P_log2) - 1;
  const int32_t* table = page_table + static_cast<size_t>(b) * max_pages;
  const int32_t* path = paths + static_cast<size_t>(b) * K;
  T* const kc = static_cast<T*>(p.k_cache);
  T* const vc = static_cast<T*>(p.v_cache);
  auto k_at = [&](int page, int slot) {
    return (static_cast<size_t>(page * p.Hkv + g) * (Pm1 + 1) + slot) * D + x;
  };
  auto v_at = [&](int page, int slot) {
    return (static_cast<size_t>(page * p.Hkv + g) * D + x) * (Pm1 + 1) + slot;
  };
  auto page_of = [&](int pos) {
    const int pg = table[pos >> P_log2];
    return (pg >= 0 && pg < p.num_pages) ? pg : -1;
  };
  for (int j = 1; j <= a; ++j) {
    const int node = path[j];
    if (node <= j || node >= K) continue;         // in place, or not a path node
    const int src = ctx + node;
    const int pg = page_of(src);
    if (pg < 0) continue;
    ks[(j - 1) * D + x] = kc[k_at(pg, src & Pm1)];
    vs[(j - 1) * D + x] = vc[v_at(pg, src & Pm1)];
  }
  for (int j = 1; j <= a; ++j) {
    const int node = path[j];
    if (node <= j || node >= K) continue;
    const int src = ctx + node, dst = ctx + j;
    const int ps = page_of(src), pd = page_of(dst);
    if (ps < 0 || pd < 0) continue;
    kc[k_at(pd, dst & Pm1)] = ks[(j - 1) * D + x];
    vc[v_at(pd, dst & Pm1)] = vs[(j - 1) * D + x];
  }
}

}  // namespace

hipError_t launch_tree_compact(const TreeCompactParams& p, hipStream_t stream) {
#define TREE_ARGS p.accept_len, p.ctx_lens, p.page_table, p.path, p.K, p.D, p.max_pages, p.P_log2, p
  const size_t lds = 2 * static_cast<size_t>(p.K - 1) * p.D * p.esz;
  if (p.esz == 4)
    hipLaunchKernelGGL(tree_compact_kernel<uint32_t>, dim3(p.Hkv, p.B), dim3(128), lds, stream,
                       TREE_ARGS);
  else
    hipLaunchKernelGGL(tree_compact_kernel<uint16_t>, dim3(p.Hkv, p.B), dim3(128), lds, stream,
                       TREE_ARGS);
#undef TREE_ARGS
  return hipGetLastError();
}

hipError_t launch_commit(const CommitParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(commit_kernel, dim3((p.B + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     stream, p.accept_len, p.out_tokens, p.B, p.K, p);
  return hipGetLastError();
}

}  // namespace sv
