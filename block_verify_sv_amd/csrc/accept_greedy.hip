// Greedy acceptance: argmax of every block row over the vocabulary, then the longest
// draft prefix matching it plus the target's correction (VFlash-FM page, caption of
// the cycle figure).
//
// Two launches.  The argmax pass has grid (vocabulary chunk, block row): each workgroup
// scans a chunk of one row with 16-byte loads (all issued before any is consumed) and
// reduces a packed 64-bit key (orderable value bits << 32 | ~index) -- so the maximum
// key is the largest value at the lowest index -- through the wave and LDS into one
// plain store per (row, chunk).  The walk pass has one wave per sequence: it reduces
// the K rows' chunk keys (an order-independent maximum), and a ballot over the lanes
// whose draft differs from the target's choice gives the accepted length.  The kernel
// boundary orders the two; the workspace carries no state between calls.  A draft tree
// uses the same argmax pass and a walk from the anchor through the tree (see below).
#include "common.hpp"
#include "internal.hpp"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kLoadsPerThread = 4;                // 16-byte loads per thread per round
constexpr int kMaxChunks = 32;                    // vocabulary chunks per row, at most

template <bool kBF16>
__device__ __forceinline__ float load_logit(const void* base, size_t i) {
  if constexpr (kBF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
  else return static_cast<const float*>(base)[i];
}

// The fields the first loads need come first as plain arguments (preloaded into SGPRs).
template <bool kBF16>
__global__ void __launch_bounds__(kThreads)
greedy_argmax_kernel(const void* logits, int32_t V, int32_t chunk, const GreedyParams p) {
  __shared__ uint64_t red[kThreads / kWave];

  const int tid = threadIdx.x;
  const int row = blockIdx.y;                     // b * K + i
  const int j0 = blockIdx.x * chunk;
  const int j1 = min(j0 + chunk, V);
  const size_t rbase = static_cast<size_t>(row) * V;

  uint64_t best = 0;
  constexpr int EPV = kBF16 ? 8 : 4;              // elements per 16-byte load
  if ((V % EPV) == 0) {
    // per round every load is issued before any is consumed; indices past the row end
    // are clamped to its last 16 bytes (in bounds) and ignored below
    for (int jr = j0; jr < j1; jr += kLoadsPerThread * kThreads * EPV) {
      u32x4 v[kLoadsPerThread];
#pragma unroll
      for (int u = 0; u < kLoadsPerThread; ++u) {
        const int j = min(jr + (tid + u * kThreads) * EPV, V - EPV);
        v[u] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(logits) +
                                               (rbase + j) * (kBF16 ? 2 : 4));
      }
#pragma unroll
      for (int u = 0; u < kLoadsPerThread; ++u) {
        const int j = jr + (tid + u * kThreads) * EPV;
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
    }
  } else {
    for (int j = j0 + tid; j < j1; j += kThreads) {
      const uint64_t key = argmax_key(load_logit<kBF16>(logits, rbase + j), static_cast<uint32_t>(j));
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
    p.keys[static_cast<size_t>(row) * p.nchunk + blockIdx.x] = m;
  }
}

constexpr int kWalkSeqs = kThreads / kWave;       // sequences per walk workgroup

__global__ void __launch_bounds__(kThreads)
greedy_walk_kernel(const unsigned long long* chunk_keys, const int32_t* drafts, int32_t B, int32_t K,
                   int32_t nchunk, const GreedyParams p) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * kWalkSeqs + (threadIdx.x >> 6);
  if (b >= B) return;                             // whole waves
  const bool in = lane < K;
  // draft k+1 (drafts[b][k]) is checked against row k's choice, k = 0 .. K-2; loaded
  // first (clamped, unconditional) so that it shares the keys' round trip
  const int32_t dl = K > 1 ? drafts[static_cast<size_t>(b) * (K - 1) + min(lane, K - 2)] : 0;
  // lane i reduces row i's chunk keys (at most kMaxChunks; plain data written by the
  // argmax pass; all loads in flight, clamped index)
  const unsigned long long* keys = chunk_keys + static_cast<size_t>(b) * K * nchunk;
  uint64_t best = 0;
  if (in) {
    uint64_t k[kMaxChunks];
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c)
      k[c] = keys[static_cast<size_t>(lane) * nchunk + min(c, nchunk - 1)];
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) best = k[c] > best ? k[c] : best;
  }
  const int32_t t = in ? static_cast<int32_t>(argmax_key_index(best)) : -1;
  const int32_t d = lane < K - 1 ? dl : 0;
  const uint64_t miss = __ballot(lane < K - 1 && d != t);
  const int a = miss ? __builtin_ctzll(miss) : K - 1;   // accepted drafts
  const int32_t corr = __shfl(t, a);
  // every store last: a store before the ballot made the compiler wait for its
  // acknowledgement before using the (long since loaded) draft token
  if (in) {
    if (p.argmax) p.argmax[static_cast<size_t>(b) * K + lane] = t;
    p.out_tokens[static_cast<size_t>(b) * K + lane] = lane < a ? d : (lane == a ? corr : -1);
  }
  if (lane == 0) p.accept_len[b] = a;
}

// Tree walk (a draft tree verified greedily: the chain rule walked from the anchor).
// One wave per sequence; lane i holds node i's greedy token, parent and draft token.
// From the anchor, a ballot over the lanes that hang under the current node, are
// numbered above it and hold its greedy token picks the lowest such lane as the next
// node.  Each step raises the node number, so the walk ends within K-1 steps whatever
// the parent array holds.
__global__ void __launch_bounds__(kThreads)
greedy_tree_walk_kernel(const unsigned long long* chunk_keys, const int32_t* drafts,
                        const int32_t* parents, int32_t B, int32_t K, int32_t nchunk,
                        const GreedyParams p) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * kWalkSeqs + (threadIdx.x >> 6);
  if (b >= B) return;                             // whole waves
  const bool in = lane < K;
  // the node's parent and draft token, loaded first (clamped, unconditional) so that
  // they share the keys' round trip
  const size_t nb0 = static_cast<size_t>(b) * (K - 1) + min(max(lane - 1, 0), max(K - 2, 0));
  const int32_t par_l = K > 1 ? parents[nb0] : -1;
  const int32_t tok_l = K > 1 ? drafts[nb0] : 0;
  const unsigned long long* keys = chunk_keys + static_cast<size_t>(b) * K * nchunk;
  uint64_t best = 0;
  if (in) {
    uint64_t k[kMaxChunks];
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c)
      k[c] = keys[static_cast<size_t>(lane) * nchunk + min(c, nchunk - 1)];
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) best = k[c] > best ? k[c] : best;
  }
  const int32_t t = in ? static_cast<int32_t>(argmax_key_index(best)) : -1;
  const bool node = lane >= 1 && lane < K;        // a draft node
  const int32_t par = node ? par_l : -1;
  const int32_t tok = node ? tok_l : 0;
  int cur = 0, a = 0;
  int32_t my_path = lane == 0 ? 0 : -1;           // lane j ends up holding path[j]
  for (int step = 1; step < K; ++step) {
    const int32_t want = __shfl(t, cur);
    const uint64_t hit = __ballot(node && lane > cur && par == cur && tok == want);
    if (!hit) break;
    cur = __builtin_ctzll(hit);
    a = step;
    if (lane == step) my_path = cur;
  }
  const int32_t next_node = __shfl(my_path, lane < 63 ? lane + 1 : 63);   // path[j+1]
  const int32_t next_tok = __shfl(tok, next_node > 0 ? next_node : 0);
  const int32_t corr = __shfl(t, cur);
  if (in) {                                        // every store last (as in the chain walk)
    const size_t o = static_cast<size_t>(b) * K + lane;
    if (p.argmax) p.argmax[o] = t;
    p.out_tokens[o] = lane < a ? next_tok : (lane == a ? corr : -1);
    p.path[o] = my_path;
  }
  if (lane == 0) p.accept_len[b] = a;
}

}  // namespace

size_t greedy_workspace_bytes(int B, int K) {
  return static_cast<size_t>(B) * K * kMaxChunks * sizeof(unsigned long long);
}

int greedy_chunk(int V, sv_dtype dtype) {
  // rounds of kLoadsPerThread 16-byte loads per thread (16 KB per workgroup), and at
  // most kMaxChunks chunks per row
  const int round = kLoadsPerThread * kThreads * (dtype == SV_BF16 ? 8 : 4);
  const int rounds = (V + round - 1) / round;
  return round * ((rounds + kMaxChunks - 1) / kMaxChunks);
}

hipError_t launch_greedy(const GreedyParams& p, sv_dtype dtype, hipStream_t stream) {
  const dim3 grid(p.nchunk, p.B * p.K);
  if (dtype == SV_BF16)
    hipLaunchKernelGGL(greedy_argmax_kernel<true>, grid, dim3(kThreads), 0, stream, p.logits, p.V,
                       p.chunk, p);
  else
    hipLaunchKernelGGL(greedy_argmax_kernel<false>, grid, dim3(kThreads), 0, stream, p.logits, p.V,
                       p.chunk, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_greedy_walk(p, stream);
}

hipError_t launch_greedy_walk(const GreedyParams& p, hipStream_t stream) {
  if (p.tree)
    hipLaunchKernelGGL(greedy_tree_walk_kernel, dim3((p.B + kWalkSeqs - 1) / kWalkSeqs),
                       dim3(kThreads), 0, stream, p.keys, p.drafts, p.parents, p.B, p.K, p.nchunk, p);
  else
    hipLaunchKernelGGL(greedy_walk_kernel, dim3((p.B + kWalkSeqs - 1) / kWalkSeqs),
                       dim3(kThreads), 0, stream, p.keys, p.drafts, p.B, p.K, p.nchunk, p);
  return hipGetLastError();
}

}  // namespace sv
