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

__global__ void __launch_bounds__(kThreads) commit_kernel(const CommitParams p) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= p.B) return;
  int a = p.accept_len[b];
  a = a < 0 ? 0 : (a > p.K - 1 ? p.K - 1 : a);
  p.next_anchor[b] = p.out_tokens[static_cast<size_t>(b) * p.K + a];
  p.ctx_lens[b] += a + 1;
}

}  // namespace

hipError_t launch_commit(const CommitParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(commit_kernel, dim3((p.B + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace sv
