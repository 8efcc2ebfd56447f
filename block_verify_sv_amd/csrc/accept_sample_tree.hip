// Sampling verification of a draft tree: recursive rejection over the children of the
// current node (the standard acceptance-rejection rule of the SpecFLASH README applied
// to the "Tree-60" draft trees of the VFlash-FM results table).
//
// At node u with children c_1 < c_2 < ... (tokens x_j drawn from draft rows q_j) the
// residual starts as r_0 = p_u; child c_j passes iff u_j < min(1, r_{j-1}(x_j) / q_j(x_j));
// a rejection leaves r_j = max(0, r_{j-1} - q_j) / Z_j with Z_j = sum_v max(0, r_{j-1} -
// q_j)(v) (p_u if Z_j = 0).  The first child that passes becomes the current node; when
// none does, the token is drawn from the last residual (p_u at a leaf).  Whether c_j
// passes depends only on (u, j), never on the path that reached u, so every test is
// decided in parallel once the normalisers are known, and the walk itself is a few
// ballots.  On a chain this is the chain rule exactly (same uniforms, same arithmetic).
//
// Launches (the tree is host data, shared by the batch, so its shape fixes the plan):
//   1. row_lse_kernel (the chain's): per-chunk (max, sum) of every target and draft row;
//   2. for j = 1 .. (largest child count - 1): tree_residual_kernel, grid (vocabulary
//      chunk, sequence x node with more than j children): the partial sums of Z_j at
//      every such node, the residual rebuilt element by element from p_u, the first j
//      draft rows and Z_1 .. Z_{j-1} (fp64);
//   3. tree_walk_kernel, one workgroup per sequence: the row log-normalisers, every
//      child's threshold and ACCEPT uniform (lane = node), then the walk from the anchor;
//   4. tree_race_kernel, grid (1024-entry chunk, sequence): the exponential race over the
//      stop node's last residual (the chain's race: RESAMPLE uniforms of the stop row,
//      with a race over p_u carried along for an all-zero residual);
//   5. tree_finish_kernel, one workgroup per sequence: the winner and the outputs.
// Kernel boundaries order everything; the workspace carries no state between calls.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"
#include "sample_device.hpp"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kZChunk = 16 * kThreads;            // vocabulary entries per residual workgroup
constexpr int kRaceChunk = 4 * kThreads;          // vocabulary entries per race workgroup
constexpr uint64_t kResample = 1ull << 32;        // RESAMPLE purpose in counter word 2

// Log-normaliser L = m/T + log sum_c s_c e^((m_c - m)/T) of row rho from the chunk partials
// (fixed order; the chain's combine).
__device__ __forceinline__ double row_norm(const float* part_m, const double* part_s, int rho,
                                           int nchunk, double it) {
  const float* pm = part_m + static_cast<size_t>(rho) * nchunk;
  const double* ps = part_s + static_cast<size_t>(rho) * nchunk;
  float m = -INFINITY;
  for (int q = 0; q < nchunk; ++q) m = fmaxf(m, pm[q]);
  double s = 0.0;
  for (int q = 0; q < nchunk; ++q)
    s += ps[q] * exp((static_cast<double>(pm[q]) - static_cast<double>(m)) * it);
  return static_cast<double>(m) * it + log(s);
}

// Z of the residual left by rejecting child node c (fixed-order sum of its partials).
__device__ __forceinline__ double z_of(const double* zpart, int b, int K, int c, int nz) {
  const double* z = zpart + (static_cast<size_t>(b) * K + c) * nz;
  double s = 0.0;
  for (int q = 0; q < nz; ++q) s += z[q];
  return s;
}

// Row index rho of target row u / draft row of node c for the row_lse partials.
__device__ __forceinline__ int target_rho(int b, int K, int u) { return b * K + u; }
__device__ __forceinline__ int draft_rho(int B, int b, int K, int c) {
  return B * K + b * (K - 1) + (c - 1);
}

// ---- 2. residual normalisers, round j: Z of the residual after rejecting the j-th child
template <bool kBF16>
__global__ void __launch_bounds__(kThreads)
tree_residual_kernel(int32_t j, int32_t n_nodes, const TreeSampleParams p) {
  __shared__ double Lp_sh, Lq_sh[kMaxBlock], Z_sh[kMaxBlock];
  __shared__ int32_t kid_sh[kMaxBlock];
  __shared__ double red[kThreads / kWave];
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x;
  const int b = blockIdx.y / n_nodes;
  const int u = p.by_count[blockIdx.y - b * n_nodes];
  const int K = p.K, V = p.V;
  const double it = p.inv_t;
  const int first = p.child_start[u];
  if (tid <= j) {                                  // lane 0: p_u; lane i: child i's row
    if (tid == 0) {
      Lp_sh = row_norm(p.part_m, p.part_s, target_rho(b, K, u), p.nchunk, it);
    } else {
      const int c = p.child_list[first + tid - 1];
      kid_sh[tid - 1] = c;
      Lq_sh[tid - 1] = row_norm(p.part_m, p.part_s, draft_rho(p.B, b, K, c), p.nchunk, it);
      if (tid < j) Z_sh[tid - 1] = z_of(p.zpart, b, K, c, p.nz);
    }
  }
  __syncthreads();
  const size_t trow = (static_cast<size_t>(b) * K + u) * V;
  double sum = 0.0;
  for (int e = 0; e < kZChunk / kThreads; ++e) {
    const int v = chunk * kZChunk + e * kThreads + tid;
    if (v >= V) break;
    const double pv = exp(static_cast<double>(logit_at<kBF16>(p.target, trow + v)) * it - Lp_sh);
    double r = pv, raw = 0.0;
    for (int i = 0; i < j; ++i) {
      const size_t qrow = (static_cast<size_t>(b) * (K - 1) + (kid_sh[i] - 1)) * V;
      const double qv = exp(static_cast<double>(logit_at<kBF16>(p.draft, qrow + v)) * it - Lq_sh[i]);
      raw = fmax(0.0, r - qv);
      if (i + 1 < j) r = Z_sh[i] > 0.0 ? raw / Z_sh[i] : pv;
    }
    sum += raw;
  }
  sum = wave_sum_f64(sum);
  if ((tid & 63) == 0) red[tid >> 6] = sum;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) t += red[w];
    p.zpart[(static_cast<size_t>(b) * K + kid_sh[j - 1]) * p.nz + chunk] = t;
  }
}

// ---- 3. the tests and the walk, one workgroup per sequence
template <bool kBF16>
__global__ void __launch_bounds__(kThreads)
tree_walk_kernel(const TreeSampleParams p) {
  __shared__ double Lrow[2 * kMaxBlock];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int K = p.K, V = p.V;
  const double it = p.inv_t;
  for (int row = tid; row < 2 * K - 1; row += kThreads)
    Lrow[row] = row_norm(p.part_m, p.part_s,
                         row < K ? target_rho(b, K, row) : draft_rho(p.B, b, K, row - K + 1),
                         p.nchunk, it);
  __syncthreads();
  if (tid >= 64) return;
  const int lane = tid;
  const int c = lane + 1;                          // the draft node this lane tests
  const bool node = c < K;
  bool pass = false;
  if (node) {
    const int u = p.parent[c];
    const int jj = p.sib[c];                      // elder siblings rejected before this test
    const int32_t x = p.tokens[static_cast<size_t>(b) * (K - 1) + (c - 1)];
    if (x >= 0 && x < V) {
      const double lp = logit_at<kBF16>(p.target, (static_cast<size_t>(b) * K + u) * V + x);
      const double lq = logit_at<kBF16>(p.draft, (static_cast<size_t>(b) * (K - 1) + (c - 1)) * V + x);
      double thr = 0.0;
      if (lp != -INFINITY) {
        if (jj == 0) {                             // against p_u: the chain's log form
          thr = exp(fmin(0.0, (lp - lq) * it - (Lrow[u] - Lrow[K + c - 1])));
        } else {
          const double pv = exp(lp * it - Lrow[u]);
          double r = pv;
          for (int i = 0; i < jj; ++i) {
            const int ci = p.child_list[p.child_start[u] + i];
            const double lqi = logit_at<kBF16>(p.draft, (static_cast<size_t>(b) * (K - 1) + (ci - 1)) * V + x);
            const double qi = exp(lqi * it - Lrow[K + ci - 1]);
            const double raw = fmax(0.0, r - qi);
            const double z = z_of(p.zpart, b, K, ci, p.nz);
            r = z > 0.0 ? raw / z : pv;
          }
          const double qc = exp(lq * it - Lrow[K + c - 1]);
          thr = r == 0.0 ? 0.0 : (qc == 0.0 ? 1.0 : fmin(1.0, r / qc));
        }
      }
      const U64x4 w = philox(p.offset, static_cast<uint64_t>(b), static_cast<uint64_t>(c), 0,
                             p.seed, 0);
      pass = to_uniform(w.x[0]) < thr;
    }
  }
  // the walk: at the current node the lowest-numbered passing child (children are
  // tested in increasing node order); node numbers only grow, so it ends within K-1 steps
  const int par = node ? p.parent[c] : -1;
  int cur = 0, a = 0;
  int32_t my_path = lane == 0 ? 0 : -1;            // lane j ends up holding path[j]
  for (int step = 1; step < K; ++step) {
    const uint64_t hit = __ballot(node && pass && par == cur);
    if (!hit) break;
    cur = __builtin_ctzll(hit) + 1;
    a = step;
    if (lane == step) my_path = cur;
  }
  const int32_t tok = node ? p.tokens[static_cast<size_t>(b) * (K - 1) + (c - 1)] : 0;
  const int32_t next_node = __shfl(my_path, lane < 63 ? lane + 1 : 63);   // path[j+1]
  const int32_t next_tok = __shfl(tok, next_node > 0 ? next_node - 1 : 0);
  if (lane < K) {
    const size_t o = static_cast<size_t>(b) * K + lane;
    if (lane != a) p.out_tokens[o] = lane < a ? next_tok : -1;   // slot a: the drawn token
    p.path[o] = my_path;
  }
  if (lane == 0) {
    p.accept_len[b] = a;
    p.stop[2 * b] = cur;
    p.stop[2 * b + 1] = p.child_count[cur];
  }
}

// ---- 4. the race over the stop node's last residual
template <bool kBF16>
__global__ void __launch_bounds__(kThreads)
tree_race_kernel(const TreeSampleParams p) {
  __shared__ double Lp_sh, Lq_sh[kMaxBlock], Z_sh[kMaxBlock];
  __shared__ int32_t kid_sh[kMaxBlock];
  __shared__ double rk[2][kThreads / kWave];
  __shared__ int32_t ri[2][kThreads / kWave];
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x;
  const int b = blockIdx.y;
  const int K = p.K, V = p.V;
  const double it = p.inv_t;
  const int u = p.stop[2 * b];
  const int m = p.stop[2 * b + 1];                 // children rejected at u
  const int first = p.child_start[u];
  if (tid <= m) {
    if (tid == 0) {
      Lp_sh = row_norm(p.part_m, p.part_s, target_rho(b, K, u), p.nchunk, it);
    } else {
      const int c = p.child_list[first + tid - 1];
      kid_sh[tid - 1] = c;
      Lq_sh[tid - 1] = row_norm(p.part_m, p.part_s, draft_rho(p.B, b, K, c), p.nchunk, it);
      if (tid < m) Z_sh[tid - 1] = z_of(p.zpart, b, K, c, p.nz);
    }
  }
  __syncthreads();
  const size_t trow = (static_cast<size_t>(b) * K + u) * V;
  const int jb = chunk * p.race_chunk + 4 * tid;
  double bk_r = INFINITY, bk_p = INFINITY;
  int32_t bi_r = 0x7FFFFFFF, bi_p = 0x7FFFFFFF;
  if (jb < V) {
    const U64x4 w = philox(p.offset, static_cast<uint64_t>(b), kResample | static_cast<uint64_t>(u),
                           static_cast<uint64_t>(jb >> 2), p.seed, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = jb + e;
      if (v >= V) break;
      const double pv = exp(static_cast<double>(logit_at<kBF16>(p.target, trow + v)) * it - Lp_sh);
      double r = pv;
      for (int i = 0; i < m; ++i) {
        const size_t qrow = (static_cast<size_t>(b) * (K - 1) + (kid_sh[i] - 1)) * V;
        const double qv = exp(static_cast<double>(logit_at<kBF16>(p.draft, qrow + v)) * it - Lq_sh[i]);
        const double raw = fmax(0.0, r - qv);
        r = (i + 1 < m) ? (Z_sh[i] > 0.0 ? raw / Z_sh[i] : pv) : raw;
      }
      const double ej = -log1p(-to_uniform(w.x[e]));
      if (r > 0.0) {
        const double k = ej / r;
        if (better(k, v, bk_r, bi_r)) { bk_r = k; bi_r = v; }
      }
      if (pv > 0.0) {
        const double k = ej / pv;
        if (better(k, v, bk_p, bi_p)) { bk_p = k; bi_p = v; }
      }
    }
  }
  block_best<kThreads>(bk_r, bi_r, bk_p, bi_p, rk, ri);
  if (tid == 0) {
    const size_t slot = (static_cast<size_t>(b) * p.race_nchunk + chunk) * 2;
    p.race_key[slot] = bk_r;
    p.race_idx[slot] = bi_r;
    p.race_key[slot + 1] = bk_p;
    p.race_idx[slot + 1] = bi_p;
  }
}

// ---- 5. the winner over every chunk, then the drawn token at slot accept_len
__global__ void __launch_bounds__(kThreads)
tree_finish_kernel(const TreeSampleParams p) {
  __shared__ double rk[2][kThreads / kWave];
  __shared__ int32_t ri[2][kThreads / kWave];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  double bk_r = INFINITY, bk_p = INFINITY;
  int32_t bi_r = 0x7FFFFFFF, bi_p = 0x7FFFFFFF;
  for (int q = tid; q < p.race_nchunk; q += kThreads) {
    const size_t slot = (static_cast<size_t>(b) * p.race_nchunk + q) * 2;
    const double k0 = p.race_key[slot], k1 = p.race_key[slot + 1];
    const int32_t i0 = p.race_idx[slot], i1 = p.race_idx[slot + 1];
    if (better(k0, i0, bk_r, bi_r)) { bk_r = k0; bi_r = i0; }
    if (better(k1, i1, bk_p, bi_p)) { bk_p = k1; bi_p = i1; }
  }
  block_best<kThreads>(bk_r, bi_r, bk_p, bi_p, rk, ri);
  if (tid == 0) {
    const int32_t token = (bk_r < INFINITY) ? bi_r : (bk_p < INFINITY ? bi_p : -1);
    p.out_tokens[static_cast<size_t>(b) * p.K + p.accept_len[b]] = token;
  }
}

}  // namespace

size_t sample_tree_workspace_bytes(int B, int K, int V) {
  const size_t rows = static_cast<size_t>(B) * (2 * K - 1);
  const size_t nchunk = (static_cast<size_t>(V) + sample_chunk(V) - 1) / sample_chunk(V);
  const size_t nz = (static_cast<size_t>(V) + kZChunk - 1) / kZChunk;
  const size_t nrace = (static_cast<size_t>(V) + kRaceChunk - 1) / kRaceChunk;
  size_t off = 0;
  off += rows * nchunk * sizeof(double);                        // part_s
  off += static_cast<size_t>(B) * K * nz * sizeof(double);      // zpart
  off += static_cast<size_t>(B) * nrace * 2 * sizeof(double);   // race_key
  off += rows * nchunk * sizeof(float);                         // part_m
  off += static_cast<size_t>(B) * nrace * 2 * sizeof(int32_t);  // race_idx
  off += static_cast<size_t>(B) * 2 * sizeof(int32_t);          // stop
  return (off + 15) & ~static_cast<size_t>(15);
}

int plan_sample_tree(TreeSampleParams& p, const int32_t* parents_host) {
  const int K = p.K;
  p.zchunk = kZChunk;
  p.nz = (p.V + kZChunk - 1) / kZChunk;
  p.race_chunk = kRaceChunk;
  p.race_nchunk = (p.V + kRaceChunk - 1) / kRaceChunk;
  p.parent[0] = -1;
  p.sib[0] = 0;
  int count[kMaxBlock] = {0};
  for (int i = 1; i < K; ++i) {
    const int par = parents_host[i - 1];
    p.parent[i] = static_cast<int8_t>(par);
    p.sib[i] = static_cast<int8_t>(count[par]);
    ++count[par];
  }
  int pos = 0;
  for (int u = 0; u < K; ++u) {
    p.child_start[u] = static_cast<int8_t>(pos);
    p.child_count[u] = static_cast<int8_t>(count[u]);
    for (int i = u + 1; i < K; ++i)
      if (parents_host[i - 1] == u) p.child_list[pos++] = static_cast<int8_t>(i);
  }
  for (int i = K; i < kMaxBlock; ++i) {
    p.parent[i] = -1;
    p.sib[i] = 0;
    p.child_start[i] = 0;
    p.child_count[i] = 0;
  }
  int nb = 0, mmax = 0;
  for (int cnt = K - 1; cnt >= 1; --cnt)        // nodes by decreasing child count
    for (int u = 0; u < K; ++u)
      if (count[u] == cnt) p.by_count[nb++] = static_cast<int8_t>(u);
  for (int u = 0; u < K; ++u) mmax = count[u] > mmax ? count[u] : mmax;
  return mmax > 1 ? mmax - 1 : 0;
}

hipError_t launch_sample_tree(const TreeSampleParams& p, int rounds, sv_dtype dtype,
                              hipStream_t stream) {
  SampleParams lse;
  lse.target = p.target;
  lse.draft = p.draft;
  lse.B = p.B;
  lse.K = p.K;
  lse.V = p.V;
  lse.chunk = sample_chunk(p.V);
  lse.nchunk = p.nchunk;
  lse.part_m = const_cast<float*>(p.part_m);
  lse.part_s = const_cast<double*>(p.part_s);
  lse.inv_t = p.inv_t;
  hipError_t e = launch_row_lse(lse, dtype, stream);
  if (e != hipSuccess) return e;
  const bool bf = dtype == SV_BF16;
  for (int j = 1; j <= rounds; ++j) {
    int n = 0;                                    // nodes with more than j children
    for (int u = 0; u < p.K; ++u) n += p.child_count[u] > j ? 1 : 0;
    const dim3 g(p.nz, p.B * n);
    if (bf) hipLaunchKernelGGL(tree_residual_kernel<true>, g, dim3(kThreads), 0, stream, j, n, p);
    else hipLaunchKernelGGL(tree_residual_kernel<false>, g, dim3(kThreads), 0, stream, j, n, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (bf) hipLaunchKernelGGL(tree_walk_kernel<true>, dim3(p.B), dim3(kThreads), 0, stream, p);
  else hipLaunchKernelGGL(tree_walk_kernel<false>, dim3(p.B), dim3(kThreads), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 gr(p.race_nchunk, p.B);
  if (bf) hipLaunchKernelGGL(tree_race_kernel<true>, gr, dim3(kThreads), 0, stream, p);
  else hipLaunchKernelGGL(tree_race_kernel<false>, gr, dim3(kThreads), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tree_finish_kernel, dim3(p.B), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sv
