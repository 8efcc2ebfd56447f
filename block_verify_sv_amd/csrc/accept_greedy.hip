// Greedy acceptance: argmax of every block row over the vocabulary, then the longest
// draft prefix matching it plus the target's correction (VFlash-FM page, caption of
// the cycle figure).
//
// One launch.  Grid (vocabulary chunk, block row).  Each workgroup scans a chunk of one
// row with 16-byte loads and reduces a packed 64-bit key (orderable value bits << 32 |
// ~index) -- so the maximum key is the largest value at the lowest index -- through the
// wave and LDS into one atomicMax per workgroup.  The last workgroup to arrive for a
// sequence (arrival counter, bumped only after the atomicMax has returned) decodes the
// K row maxima, walks the draft prefix, writes the outputs and returns its keys and
// counter to zero for the next call.
#include "common.hpp"
#include "internal.hpp"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kLoadsPerThread = 4;                // 16-byte loads per thread per chunk

template <bool kBF16>
__device__ __forceinline__ float load_logit(const void* base, size_t i) {
  if constexpr (kBF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
  else return static_cast<const float*>(base)[i];
}

template <bool kBF16>
__global__ void __launch_bounds__(kThreads) greedy_kernel(const GreedyParams p) {
  __shared__ uint64_t red[kThreads / kWave];
  __shared__ int32_t tok[kMaxBlock];
  __shared__ int32_t acc_len;
  __shared__ bool is_last;

  const int tid = threadIdx.x;
  const int row = blockIdx.y;                     // b * K + i
  const int b = row / p.K;
  const int j0 = blockIdx.x * p.chunk;
  const int j1 = min(j0 + p.chunk, p.V);
  const size_t rbase = static_cast<size_t>(row) * p.V;

  uint64_t best = 0;
  constexpr int EPV = kBF16 ? 8 : 4;              // elements per 16-byte load
  if ((p.V % EPV) == 0) {
    // every load of the chunk is issued before any is consumed
    u32x4 v[kLoadsPerThread];
#pragma unroll
    for (int u = 0; u < kLoadsPerThread; ++u) {
      const int j = j0 + (tid + u * kThreads) * EPV;
      v[u] = j < j1 ? *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.logits) +
                                                     (rbase + j) * (kBF16 ? 2 : 4))
                    : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kLoadsPerThread; ++u) {
      const int j = j0 + (tid + u * kThreads) * EPV;
      if (j >= j1) continue;
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        float x;
        if constexpr (kBF16) x = bf16_to_f32(static_cast<uint16_t>(v[u][e >> 1] >> (16 * (e & 1))));
        else x = __uint_as_float(v[u][e]);
        const uint64_t key = argmax_key(x, static_cast<uint32_t>(j + e));
        best = key > best ? key : best;
      }
    }
  } else {
    for (int j = j0 + tid; j < j1; j += kThreads) {
      const uint64_t key = argmax_key(load_logit<kBF16>(p.logits, rbase + j), static_cast<uint32_t>(j));
      best = key > best ? key : best;
    }
  }
  best = wave_max_u64(best);
  if ((tid & 63) == 0) red[tid >> 6] = best;
  __syncthreads();
  if (tid == 0) {
    uint64_t m = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / kWave; ++w) m = red[w] > m ? red[w] : m;
    // The keys only ever move through device-scope atomics, so no fence is needed: the
    // returning atomicMax has been performed at the coherence point before the arrival
    // counter is bumped, and the last arrival reads the keys atomically.
    const unsigned long long before = __hip_atomic_fetch_max(
        &p.keys[row], static_cast<unsigned long long>(m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned prev = __hip_atomic_fetch_add(&p.counters[b], before == ~0ull ? 0u : 1u,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = prev == static_cast<unsigned>(p.nchunk * p.K - 1);
  }
  __syncthreads();
  if (!is_last) return;

  // ---- last workgroup of sequence b: decode maxima, walk the draft prefix
  const int K = p.K;
  if (tid < K) {
    // read-and-clear in one RMW: it returns the latest value in the key's modification
    // order and leaves the key zeroed for the next call
    unsigned long long* kp = &p.keys[static_cast<size_t>(b) * K + tid];
    const uint64_t key = __hip_atomic_exchange(kp, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int32_t t = static_cast<int32_t>(argmax_key_index(key));
    tok[tid] = t;
    if (p.argmax) p.argmax[static_cast<size_t>(b) * K + tid] = t;
  }
  __syncthreads();
  const int32_t* dr = p.drafts + static_cast<size_t>(b) * (K - 1);
  if (tid == 0) {
    int a = 0;
    while (a < K - 1 && dr[a] == tok[a]) ++a;
    acc_len = a;
    p.accept_len[b] = a;
    __hip_atomic_store(&p.counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (tid < K) {
    const int a = acc_len;
    p.out_tokens[static_cast<size_t>(b) * K + tid] = tid < a ? dr[tid] : (tid == a ? tok[a] : -1);
  }
}

}  // namespace

size_t greedy_workspace_bytes(int B, int K) {
  const size_t keys = static_cast<size_t>(B) * K * sizeof(unsigned long long);
  return keys + static_cast<size_t>(B) * sizeof(unsigned int);
}

int greedy_chunk(int V, sv_dtype dtype) {
  (void)V;
  // 16 KB of logits per workgroup: kLoadsPerThread 16-byte loads per thread
  return kLoadsPerThread * kThreads * (dtype == SV_BF16 ? 8 : 4);
}

hipError_t launch_greedy(const GreedyParams& p, sv_dtype dtype, hipStream_t stream) {
  const dim3 grid(p.nchunk, p.B * p.K);
  if (dtype == SV_BF16)
    hipLaunchKernelGGL(greedy_kernel<true>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(greedy_kernel<false>, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sv
