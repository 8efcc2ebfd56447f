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
//   2. tree_norm_kernel: every row's log-normaliser, one wave per row, into a table;
//   3. for j = 1 .. (largest child count - 1): tree_residual_kernel, grid (1024-entry
//      vocabulary chunk, sequence x node with more than j children): the residual after
//      the j-th child, max(0, rhat_{j-1} - q_j), stored per element in fp64 (one row per
//      branching node, updated in place pass after pass) and its partial sums, which the
//      next pass folds into Z_j; after the last pass tree_z_kernel folds the last ones;
//   4. tree_walk_kernel, one wave per sequence: every child's threshold and ACCEPT uniform
//      (lane = node), then the walk from the anchor;
//   5. tree_race_kernel, grid (1024-entry chunk, sequence): the exponential race over the
//      stop node's last residual (the chain's race: RESAMPLE uniforms of the stop row,
//      with a race over p_u carried along for an all-zero residual);
//   6. tree_finish_kernel, one workgroup per sequence: the winner and the outputs.
// Kernel boundaries order everything; the workspace carries no state between calls.
// Every reduction runs in a fixed order, so results are bitwise reproducible.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"
#include "sample_device.hpp"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kZChunk = 4 * kThreads;             // vocabulary entries per residual workgroup
constexpr int kRaceChunk = 4 * kThreads;          // vocabulary entries per race workgroup
constexpr uint64_t kResample = 1ull << 32;        // RESAMPLE purpose in counter word 2

// Row index rho of target row u / draft row of node c for the row_lse partials.
__device__ __forceinline__ int target_rho(int b, int K, int u) { return b * K + u; }
__device__ __forceinline__ int draft_rho(int B, int b, int K, int c) {
  return B * K + b * (K - 1) + (c - 1);
}

// ---- 2. every row's log-normaliser L = m/T + log sum_c s_c e^((m_c - m)/T), one wave per
// row (lanes stride over the chunk partials; fixed shuffle order)
__global__ void __launch_bounds__(kThreads)
tree_norm_kernel(int32_t rows, const TreeSampleParams p) {
  const int lane = threadIdx.x & 63;
  const int rho = blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6);
  if (rho >= rows) return;                         // whole waves
  const float* pm = p.part_m + static_cast<size_t>(rho) * p.nchunk;
  const double* ps = p.part_s + static_cast<size_t>(rho) * p.nchunk;
  float m = -INFINITY;
  for (int q = lane; q < p.nchunk; q += kWave) m = fmaxf(m, pm[q]);
  m = wave_max(m);
  double s = 0.0;
  for (int q = lane; q < p.nchunk; q += kWave)
    s += ps[q] * exp((static_cast<double>(pm[q]) - static_cast<double>(m)) * p.inv_t);
  s = wave_sum_f64(s);
  if (lane == 0) p.lnorm[rho] = static_cast<double>(m) * p.inv_t + log(s);
}

// ---- 3a. residual pass j at every node with more than j children: the residual after
// rejecting the j-th child, raw_j = max(0, rhat_{j-1} - q_j), stored per element (fp64) for
// the next pass, and its partial sums.  rhat_0 = p_u; rhat_{j-1} = raw_{j-1} / Z_{j-1}
// (p_u if Z_{j-1} = 0), with Z_{j-1} folded here from the previous pass's partial sums.
template <bool kBF16>
__global__ void __launch_bounds__(kThreads)
tree_residual_kernel(int32_t j, int32_t n_nodes, const TreeSampleParams p) {
  __shared__ double zprev_sh;
  __shared__ double red[kThreads / kWave];
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x;
  const int b = blockIdx.y / n_nodes;
  const int u = p.by_count[blockIdx.y - b * n_nodes];
  const int K = p.K, V = p.V;
  const double it = p.inv_t;
  const int first = p.child_start[u];
  const int c = p.child_list[first + j - 1];       // the child this pass subtracts
  const double Lp = p.lnorm[target_rho(b, K, u)];
  const double Lq = p.lnorm[draft_rho(p.B, b, K, c)];
  double* buf = p.resid + (static_cast<size_t>(b) * p.nbranch + p.branch_slot[u]) * V;
  const size_t trow = (static_cast<size_t>(b) * K + u) * V;
  const size_t qrow = (static_cast<size_t>(b) * (K - 1) + (c - 1)) * V;
  // this thread's elements are loaded before the fold of Z_{j-1}, so the two round trips
  // overlap (clamped, in-bounds indices; elements past V are dropped below)
  constexpr int EPT = kZChunk / kThreads;
  float xq[EPT], xp[EPT];
  double rb[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int v = min(chunk * kZChunk + e * kThreads + tid, V - 1);
    xq[e] = logit_at<kBF16>(p.draft, qrow + v);
    if (j == 1) xp[e] = logit_at<kBF16>(p.target, trow + v);
    else rb[e] = buf[v];
  }
  if (j > 1 && tid < kWave) {                      // Z_{j-1}, from the previous pass
    const int cp = p.child_list[first + j - 2];
    const double* z = p.zpart + (static_cast<size_t>(b) * K + cp) * p.nz;
    double s = 0.0;
    for (int q = tid; q < p.nz; q += kWave) s += z[q];
    s = wave_sum_f64(s);
    if (tid == 0) {
      zprev_sh = s;
      if (chunk == 0) p.ztab[static_cast<size_t>(b) * K + cp] = s;
    }
  }
  __syncthreads();
  const double zp = j > 1 ? zprev_sh : 1.0;
  if (j > 1 && !(zp > 0.0)) {                      // Z_{j-1} = 0: the residual restarts at p_u
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      xp[e] = logit_at<kBF16>(p.target, trow + min(chunk * kZChunk + e * kThreads + tid, V - 1));
  }
  const bool from_p = j == 1 || !(zp > 0.0);
  double sum = 0.0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int v = chunk * kZChunk + e * kThreads + tid;
    if (v < V) {
      const double r = from_p ? exp(static_cast<double>(xp[e]) * it - Lp) : rb[e] / zp;
      const double qv = exp(static_cast<double>(xq[e]) * it - Lq);
      const double raw = fmax(0.0, r - qv);
      buf[v] = raw;
      sum += raw;
    }
  }
  sum = wave_sum_f64(sum);
  if ((tid & 63) == 0) red[tid >> 6] = sum;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) t += red[w];
    p.zpart[(static_cast<size_t>(b) * K + c) * p.nz + chunk] = t;
  }
}

// ---- 3b. after the last pass: Z of the last subtracted child of every branching node
// (the earlier ones were folded by the passes), one wave per (sequence, node)
__global__ void __launch_bounds__(kWave)
tree_z_kernel(int32_t n_nodes, const TreeSampleParams p) {
  const int lane = threadIdx.x;
  const int b = blockIdx.x / n_nodes;
  const int u = p.by_count[blockIdx.x - b * n_nodes];
  const int c = p.child_list[p.child_start[u] + p.child_count[u] - 2];
  const double* z = p.zpart + (static_cast<size_t>(b) * p.K + c) * p.nz;
  double s = 0.0;
  for (int q = lane; q < p.nz; q += kWave) s += z[q];
  s = wave_sum_f64(s);
  if (lane == 0) p.ztab[static_cast<size_t>(b) * p.K + c] = s;
}

// ---- 4. the tests and the walk, one wave per sequence
template <bool kBF16>
__global__ void __launch_bounds__(kWave)
tree_walk_kernel(const TreeSampleParams p) {
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int K = p.K, V = p.V;
  const double it = p.inv_t;
  const double* L = p.lnorm;
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
          thr = exp(fmin(0.0, (lp - lq) * it - (L[target_rho(b, K, u)] -
                                                 L[draft_rho(p.B, b, K, c)])));
        } else {
          const double pv = exp(lp * it - L[target_rho(b, K, u)]);
          double r = pv;
#pragma unroll 4
          for (int i = 0; i < jj; ++i) {
            const int ci = p.child_list[p.child_start[u] + i];
            const double lqi = logit_at<kBF16>(p.draft, (static_cast<size_t>(b) * (K - 1) + (ci - 1)) * V + x);
            const double qi = exp(lqi * it - L[draft_rho(p.B, b, K, ci)]);
            const double raw = fmax(0.0, r - qi);
            const double z = p.ztab[static_cast<size_t>(b) * K + ci];
            r = z > 0.0 ? raw / z : pv;
          }
          const double qc = exp(lq * it - L[draft_rho(p.B, b, K, c)]);
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

// ---- 5. the race over the stop node's last residual
template <bool kBF16>
__global__ void __launch_bounds__(kThreads)
tree_race_kernel(const TreeSampleParams p) {
  __shared__ double rk[2][kThreads / kWave];
  __shared__ int32_t ri[2][kThreads / kWave];
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x;
  const int b = blockIdx.y;
  const int K = p.K, V = p.V;
  const double it = p.inv_t;
  const int u = p.stop[2 * b];
  const int m = p.stop[2 * b + 1];                 // children rejected at u
  const double Lp = p.lnorm[target_rho(b, K, u)];
  const int c = m > 0 ? p.child_list[p.child_start[u] + m - 1] : 1;   // the last one
  const double Lq = m > 0 ? p.lnorm[draft_rho(p.B, b, K, c)] : 0.0;
  const double zp = m > 1 ? p.ztab[static_cast<size_t>(b) * K + p.child_list[p.child_start[u] + m - 2]]
                          : 1.0;
  const bool from_buf = m > 1 && zp > 0.0;         // rhat_{m-1} from the stored residual
  const double* buf = p.resid + (static_cast<size_t>(b) * p.nbranch + p.branch_slot[u]) * V;
  const size_t trow = (static_cast<size_t>(b) * K + u) * V;
  const size_t qrow = (static_cast<size_t>(b) * (K - 1) + (c - 1)) * V;
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
      const double pv = exp(static_cast<double>(logit_at<kBF16>(p.target, trow + v)) * it - Lp);
      double r = pv;
      if (m > 0) {
        const double rh = from_buf ? buf[v] / zp : pv;
        const double qv = exp(static_cast<double>(logit_at<kBF16>(p.draft, qrow + v)) * it - Lq);
        r = fmax(0.0, rh - qv);
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

// ---- 6. the winner over every chunk, then the drawn token at slot accept_len
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
  off += static_cast<size_t>(B) * (K / 2) * V * sizeof(double); // resid: at most K/2 branching nodes
  off += static_cast<size_t>(B) * nrace * 2 * sizeof(double);   // race_key
  off += rows * nchunk * sizeof(float);                         // part_m
  off = (off + 7) & ~static_cast<size_t>(7);
  off += rows * sizeof(double);                                 // lnorm
  off += static_cast<size_t>(B) * K * sizeof(double);           // ztab
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
  int nbr = 0;
  for (int u = 0; u < kMaxBlock; ++u) p.branch_slot[u] = 0;
  for (int u = 0; u < K; ++u)
    if (count[u] > 1) p.branch_slot[u] = static_cast<int8_t>(nbr++);
  p.nbranch = nbr > 0 ? nbr : 1;
  int nb = 0, mmax = 0;
  for (int cnt = K - 1; cnt >= 1; --cnt)        // nodes by decreasing child count
    for (int u = 0; u < K; ++u)
      if (count[u] == cnt) p.by_count[nb++] = static_cast<int8_t>(u);
  for (int u = 0; u < K; ++u) mmax = count[u] > mmax ? count[u] : mmax;
  return mmax > 1 ? mmax - 1 : 0;
}

hipError_t launch_sample_tree(const TreeSampleParams& p, int rounds, sv_dtype dtype,
                              hipStream_t stream) {
  SampleParams lse{};
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
  const int rows = p.B * (2 * p.K - 1);
  hipLaunchKernelGGL(tree_norm_kernel, dim3((rows + kThreads / kWave - 1) / (kThreads / kWave)),
                     dim3(kThreads), 0, stream, rows, p);
  e = hipGetLastError();
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
  if (rounds > 0) {
    int n = 0;                                    // branching nodes
    for (int u = 0; u < p.K; ++u) n += p.child_count[u] > 1 ? 1 : 0;
    hipLaunchKernelGGL(tree_z_kernel, dim3(p.B * n), dim3(kWave), 0, stream, n, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (bf) hipLaunchKernelGGL(tree_walk_kernel<true>, dim3(p.B), dim3(kWave), 0, stream, p);
  else hipLaunchKernelGGL(tree_walk_kernel<false>, dim3(p.B), dim3(kWave), 0, stream, p);
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
