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
// Launches (the tree is host data, shared by the batch, so its shape fixes the plan and
// the host hands every kernel flat tables of it):
//   1. tree_row_norm_kernel: (max, sum) of each quarter of every target and draft row,
//      which the later kernels fold into the row's log-normaliser;
//   2. for j = 1 .. (largest child count - 1): tree_residual_kernel, grid (1024-entry
//      vocabulary chunk, sequence x node with more than j children): the residual after
//      the j-th child, max(0, rhat_{j-1} - q_j), stored per element in fp64 (one row per
//      branching node, updated in place pass after pass) and its partial sums, which the
//      next pass folds into Z_j.  The first pass also writes every row's normaliser into
//      a table, and each pass writes q_j at the tokens of c_j's younger siblings.
//      When the workgroups of the nodes with three or more children fit the device at
//      once, every pass runs instead as one launch, tree_residual_chain_kernel, whose
//      workgroups keep their residual entries in registers and wait on each other's
//      published partial sums (bounded waits);
//   3. tree_walk_kernel, one workgroup per sequence: its other waves gather the row
//      normalisers, the residual normalisers (folding the ones no later pass folded) and
//      every node's elder siblings' probabilities of its token while wave 0 loads its
//      node's own logits; then wave 0 computes every threshold and its ACCEPT uniform
//      (lane = node), walks from the anchor with ballots, and writes the stop node's
//      record for the race;
//   4. tree_race_kernel, grid (1024-entry chunk, sequence): the exponential race over the
//      stop node's last residual (the chain's race: RESAMPLE uniforms of the stop row,
//      with a race over p_u carried along for an all-zero residual).  Each chunk
//      publishes its winners into slots the first launch left empty; the last chunk
//      workgroup of each sequence (started after the others by in-order dispatch) waits,
//      bounded, for its sequence's slots, reduces them and writes the drawn token.
// Kernel boundaries order everything else; the workspace carries no state between calls.
// Every reduction runs in a fixed order, so results are bitwise reproducible.
#include <math.h>

#include <atomic>

#include "common.hpp"
#include "internal.hpp"
#include "sample_device.hpp"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kNormSplit = 4;                    // workgroups per row of the normaliser pass
constexpr int kNormThreads = 512;
constexpr int kNormLoads = 10;                    // 16-byte loads in flight per thread (a
                                                  // quarter of a bf16 row of 152k in one round)
constexpr int kWalkThreads = 1024;                // wave 0 walks, the others gather
constexpr int kZChunk = 4 * kThreads;             // vocabulary entries per residual workgroup
constexpr int kRaceThreads = 256;
constexpr int kRaceChunk = 4 * kRaceThreads;      // vocabulary entries per race workgroup
constexpr uint64_t kResample = 1ull << 32;        // RESAMPLE purpose in counter word 2
constexpr int kPollLoads = 3;                     // slot loads per lane in flight in one poll
constexpr int kMaxDevices = 64;                   // devices whose residency is cached

// Row index rho of target row u / draft row of node c in the normaliser table.
__device__ __forceinline__ int target_rho(int b, int K, int u) { return b * K + u; }
__device__ __forceinline__ int draft_rho(int B, int b, int K, int c) {
  return B * K + b * (K - 1) + (c - 1);
}

// ---- 1. row log-normalisers L = m/T + log sum_v e^((x_v - m)/T), each row in
// kNormSplit contiguous parts of one workgroup each.  A thread keeps a running maximum
// (fp32, raw logits) and a sum of hardware exp2 terms relative to it (fp64; rescaled in
// fp64 when the maximum moves) over a fixed set of elements; the threads' pairs are
// combined in a fixed order into the part's (m, s).  The consumers fold a row's parts
// (fold_lnorm).  -inf logits contribute nothing.
template <bool kBF16>
__global__ void __launch_bounds__(kNormThreads)
tree_row_norm_kernel(const void* target, const void* draft, int32_t B, int32_t K, int32_t V,
                     const TreeSampleParams p) {
  __shared__ float red_m[kNormThreads / kWave];
  __shared__ double red_s[kNormThreads / kWave];
  const int tid = threadIdx.x;
  const int part = blockIdx.x;
  const int rho = blockIdx.y;
  const int nt = B * K;
  constexpr int ESZ = kBF16 ? 2 : 4;
  constexpr int EPL = 16 / ESZ;                    // elements per 16-byte load
  const char* row = rho < nt
                        ? static_cast<const char*>(target) + static_cast<size_t>(rho) * V * ESZ
                        : static_cast<const char*>(draft) + static_cast<size_t>(rho - nt) * V * ESZ;
  const double it = p.inv_t;
  const float c2 = static_cast<float>(it * 1.4426950408889634);
  float m = -INFINITY;
  double s = 0.0;
  auto absorb = [&](const float* x, int n) {       // n values (invalid ones are -inf)
    float lm = -INFINITY;
    for (int e = 0; e < n; ++e) lm = fmaxf(lm, x[e]);
    if (lm > m) {                                  // the running maximum moves
      s = m == -INFINITY ? 0.0 : s * exp((static_cast<double>(m) - static_cast<double>(lm)) * it);
      m = lm;
    }
    const float mref = m == -INFINITY ? 0.0f : m;
    for (int e = 0; e < n; ++e) s += static_cast<double>(fast_exp2((x[e] - mref) * c2));
  };
  if (V % EPL == 0) {
    // every load of a round is issued before any is consumed (clamped, in-bounds
    // indices; those past the part's end are masked afterwards); non-temporal: the rows
    // stream through once here (Tree-60 call 96.2 -> 94.8 us measured)
    const int nvec = V / EPL;
    const int span = (nvec + kNormSplit - 1) / kNormSplit;
    const int v0 = part * span, v1 = min(v0 + span, nvec);
    for (int base = v0; base < v1; base += kNormLoads * kNormThreads) {
      u32x4 w[kNormLoads];
#pragma unroll
      for (int u = 0; u < kNormLoads; ++u) {
        const int i = min(base + u * kNormThreads + tid, v1 - 1);
        w[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + static_cast<size_t>(i) * 16));
      }
#pragma unroll
      for (int u = 0; u < kNormLoads; ++u) {
        const bool ok = base + u * kNormThreads + tid < v1;
        float x[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          float v;
          if constexpr (kBF16) v = bf16_to_f32(static_cast<uint16_t>(w[u][e >> 1] >> (16 * (e & 1))));
          else v = __uint_as_float(w[u][e]);
          x[e] = ok ? v : -INFINITY;
        }
        absorb(x, EPL);
      }
    }
  } else {                                         // rows not 16-byte aligned: element loads
    const int span = (V + kNormSplit - 1) / kNormSplit;
    const int v0 = part * span, v1 = min(v0 + span, V);
    constexpr int kE = 4 * kNormLoads;
    for (int base = v0; base < v1; base += kE * kNormThreads) {
      float x[kE];
#pragma unroll
      for (int u = 0; u < kE; ++u) x[u] = logit_at<kBF16>(row, min(base + u * kNormThreads + tid, v1 - 1));
#pragma unroll
      for (int u = 0; u < kE; ++u)
        if (base + u * kNormThreads + tid >= v1) x[u] = -INFINITY;
      absorb(x, kE);
    }
  }
  // the part's maximum, then every thread's sum scaled to it (fp64, fixed order)
  float mb = wave_max(m);
  if ((tid & 63) == 0) red_m[tid >> 6] = mb;
  __syncthreads();
  mb = red_m[0];
#pragma unroll
  for (int w = 1; w < kNormThreads / kWave; ++w) mb = fmaxf(mb, red_m[w]);
  double t = m == -INFINITY ? 0.0 : s * exp((static_cast<double>(m) - static_cast<double>(mb)) * it);
  t = wave_sum_f64(t);
  if ((tid & 63) == 0) red_s[tid >> 6] = t;
  __syncthreads();
  if (tid == 0) {
    double S = 0.0;
#pragma unroll
    for (int w = 0; w < kNormThreads / kWave; ++w) S += red_s[w];
    p.part_m[static_cast<size_t>(rho) * kNormSplit + part] = mb;
    p.part_s[static_cast<size_t>(rho) * kNormSplit + part] = S;
  }
  // every partial-sum slot starts empty (the fused residual passes wait on them)
  const size_t slots = static_cast<size_t>(B) * K * p.nz;
  const size_t stride = static_cast<size_t>(gridDim.x) * gridDim.y * kNormThreads;
  for (size_t i = (static_cast<size_t>(blockIdx.y) * gridDim.x + part) * kNormThreads + tid;
       i < slots; i += stride)
    reinterpret_cast<uint64_t*>(p.zpart)[i] = kSlotEmpty;
  // and so does every race slot (each sequence's last race workgroup waits on them)
  const size_t rslots = static_cast<size_t>(B) * p.race_nchunk * 2;
  for (size_t i = (static_cast<size_t>(blockIdx.y) * gridDim.x + part) * kNormThreads + tid;
       i < rslots; i += stride) {
    reinterpret_cast<uint64_t*>(p.race_key)[i] = kSlotEmpty;
    p.race_idx[i] = kIdxEmpty;
  }
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = tid; i < B; i += kNormThreads) p.fail[i] = 0;
}

// A row's log-normaliser from its kNormSplit parts (fixed order, fp64).
__device__ __forceinline__ double fold_lnorm(const TreeSampleParams& p, int rho) {
  const float* pm = p.part_m + static_cast<size_t>(rho) * kNormSplit;
  const double* ps = p.part_s + static_cast<size_t>(rho) * kNormSplit;
  float m = pm[0];
#pragma unroll
  for (int k = 1; k < kNormSplit; ++k) m = fmaxf(m, pm[k]);
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < kNormSplit; ++k)
    if (pm[k] != -INFINITY) s += ps[k] * exp((static_cast<double>(pm[k]) - static_cast<double>(m)) * p.inv_t);
  return static_cast<double>(m) * p.inv_t + log(s);
}

// Pass-node word: the node u of a residual pass, the child c it subtracts, the child cp
// subtracted by the previous pass (0xFF on the first) and u's residual row.
__device__ __forceinline__ int pn_u(int32_t w) { return w & 0xFF; }
__device__ __forceinline__ int pn_c(int32_t w) { return (w >> 8) & 0xFF; }
__device__ __forceinline__ int pn_cp(int32_t w) { return (w >> 16) & 0xFF; }
__device__ __forceinline__ int pn_slot(int32_t w) { return (w >> 24) & 0xFF; }

// ---- 2. residual pass j at every node with more than j children: the residual after
// rejecting the j-th child, raw_j = max(0, rhat_{j-1} - q_j), stored per element (fp64) for
// the next pass, and its partial sums.  rhat_0 = p_u; rhat_{j-1} = raw_{j-1} / Z_{j-1}
// (p_u if Z_{j-1} = 0), with Z_{j-1} folded here from the previous pass's partial sums.
// The pass's nodes are words off .. off+n_nodes-1 of the pass table: one scalar load
// gives everything the element loads need.
template <bool kBF16>
__global__ void __launch_bounds__(kThreads)
tree_residual_kernel(int32_t j, int32_t off, int32_t n_nodes, const TreeSampleParams p) {
  __shared__ double zprev_sh;
  __shared__ double lsh_pq[2];
  __shared__ double red[kThreads / kWave];
  __shared__ int32_t tok_sh[kMaxBlock];            // every node's token (node 0: none)
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x;
  const int b = blockIdx.y / n_nodes;
  const int32_t w = p.pass_node[off + blockIdx.y - b * n_nodes];
  const int u = pn_u(w), c = pn_c(w), cp = pn_cp(w);
  const int K = p.K, V = p.V;
  const double it = p.inv_t;
  double* buf = p.resid + (static_cast<size_t>(b) * p.nbranch + pn_slot(w)) * V;
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
  if (tid < p.K - 1) tok_sh[tid + 1] = p.tokens[static_cast<size_t>(b) * (p.K - 1) + tid];
  // row normalisers: the first pass folds its two rows from the parts (two lanes, shared
  // through LDS) and its first workgroup writes every row's into the table the later
  // kernels read
  if (j == 1) {
    if (tid < 2) lsh_pq[tid] = fold_lnorm(p, tid == 0 ? target_rho(b, K, u) : draft_rho(p.B, b, K, c));
    if (chunk == 0 && blockIdx.y == 0) {
      const int rows = p.B * (2 * K - 1);
      for (int r = tid; r < rows; r += kThreads) p.lnorm[r] = fold_lnorm(p, r);
    }
  }
  if (j > 1 && tid < kWave) {                      // Z_{j-1}, from the previous pass
    const double* z = p.zpart + (static_cast<size_t>(b) * K + cp) * p.nz;
    double sz = 0.0;
    for (int q = tid; q < p.nz; q += kWave) sz += z[q];
    sz = wave_sum_f64(sz);
    if (tid == 0) {
      zprev_sh = sz;
      if (chunk == 0) p.ztab[static_cast<size_t>(b) * K + cp] = sz;
    }
  }
  __syncthreads();
  const double Lp = j == 1 ? lsh_pq[0] : p.lnorm[target_rho(b, K, u)];
  const double Lq = j == 1 ? lsh_pq[1] : p.lnorm[draft_rho(p.B, b, K, c)];
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
  // q_c at the tokens of c's younger siblings that fall in this chunk (the walk's
  // threshold of sibling s after rejecting c needs it): lane s of wave 0 (same arithmetic
  // as the elements above)
  if (tid < K && ((p.younger[c] >> tid) & 1u)) {
    const int xs = tok_sh[tid];
    if (xs >= chunk * kZChunk && xs < min((chunk + 1) * kZChunk, V))
      p.qpair[(static_cast<size_t>(b) * K + tid) * kMaxBlock + c] =
          exp(static_cast<double>(logit_at<kBF16>(p.draft, qrow + xs)) * it - Lq);
  }
  sum = wave_sum_f64(sum);
  if ((tid & 63) == 0) red[tid >> 6] = sum;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
#pragma unroll
    for (int q = 0; q < kThreads / kWave; ++q) t += red[q];
    p.zpart[(static_cast<size_t>(b) * K + c) * p.nz + chunk] = t;
  }
}

// ---- 2b. every residual pass of every branching node in one launch, used when the
// workgroups of the nodes with three or more children fit the device at once (the host
// checks; they come first in workgroup order, so in-order dispatch makes them resident
// together).  Workgroup (pair of chunks, node x sequence) keeps its 2,048 entries of the
// node's residual in registers from pass to pass, so each row is read once and written
// once.  The only data crossing workgroups is each pass's per-chunk partial sums, and
// each is its own ready flag: the normaliser pass fills every slot with a
// signalling-NaN pattern that no arithmetic produces (fmax(0, .) never yields a NaN
// either), a workgroup publishes a sum with an agent-scope atomic store, and wave 0 of
// every workgroup of the node re-reads the previous pass's slots with agent-scope
// atomic loads until none holds the pattern.  Every awaited workgroup is running; the
// wait is bounded all the same (the call's wait limit of polls), so every wave ends.  Every element
// operation, sum and summation order is tree_residual_kernel's, and the normalisers are
// folded by the same function, so the two paths give the same bits.
template <bool kBF16>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
tree_residual_chain_kernel(int32_t off, const TreeSampleParams p) {
  __shared__ double zprev_sh;
  __shared__ double red[2][kThreads / kWave];
  __shared__ double ln_sh[kMaxBlock];             // L of target row u, then of c_1, c_2, ...
  __shared__ int32_t tok_sh[kMaxBlock];
  constexpr int EPT = kZChunk / kThreads;         // entries per thread and chunk
  constexpr int E2 = 2 * EPT;
  const int tid = threadIdx.x;
  const int pair = blockIdx.x;
  const int node = blockIdx.y / p.B;              // node-major: the most children first
  const int b = blockIdx.y - node * p.B;
  const int32_t w = p.pass_node[off + node];      // the node's first-pass word
  const int u = pn_u(w);
  const int K = p.K, V = p.V, nz = p.nz;
  const int m = p.child_count[u];
  const int cs = p.child_start[u];
  const double it = p.inv_t;
  double* buf = p.resid + (static_cast<size_t>(b) * p.nbranch + pn_slot(w)) * V;
  const size_t trow = (static_cast<size_t>(b) * K + u) * V;
  const int base = pair * 2 * kZChunk;
  // entry e: chunk 2*pair + e / EPT, the same entry of that chunk as in the per-pass kernel
  auto vidx = [&](int e) { return base + (e / EPT) * kZChunk + (e % EPT) * kThreads + tid; };
  auto qrow_of = [&](int c) { return (static_cast<size_t>(b) * (K - 1) + (c - 1)) * V; };
  // this workgroup's entries of a row: off one address with immediate offsets when the
  // pair lies wholly inside the row, else at clamped indices
  const bool whole = base + 2 * kZChunk <= V;
  auto load_row = [&](float (&x)[E2], const void* src, size_t row) {
    if (whole) {
      const size_t at = row + base + tid;
#pragma unroll
      for (int e = 0; e < E2; ++e)
        x[e] = logit_at<kBF16>(src, at + (e / EPT) * kZChunk + (e % EPT) * kThreads);
    } else {
#pragma unroll
      for (int e = 0; e < E2; ++e) x[e] = logit_at<kBF16>(src, row + min(vidx(e), V - 1));
    }
  };
  double rb[E2], qv[E2];
  float xq[E2];
  {
    float xp[E2];
    load_row(xp, p.target, trow);
    load_row(xq, p.draft, qrow_of(p.child_list[cs]));
    if (tid < K - 1) tok_sh[tid + 1] = p.tokens[static_cast<size_t>(b) * (K - 1) + tid];
    if (tid < m)                                  // this node's normalisers, one lane each
      ln_sh[tid] = fold_lnorm(p, tid == 0 ? target_rho(b, K, u)
                                          : draft_rho(p.B, b, K, p.child_list[cs + tid - 1]));
    // the table the later kernels read, from the last workgroup (the fewest passes)
    if (blockIdx.x == gridDim.x - 1 && blockIdx.y == gridDim.y - 1) {
      const int rows = p.B * (2 * K - 1);
      for (int r = tid; r < rows; r += kThreads) p.lnorm[r] = fold_lnorm(p, r);
    }
    __syncthreads();
    const double Lp = ln_sh[0], Lq = ln_sh[1];
#pragma unroll
    for (int e = 0; e < E2; ++e) {                // pass 1: the residual from p_u
      rb[e] = fmax(0.0, exp(static_cast<double>(xp[e]) * it - Lp) -
                            exp(static_cast<double>(xq[e]) * it - Lq));
      __builtin_amdgcn_sched_barrier(0);          // one entry's exponentials at a time
    }
  }
  // the pass-j sums of the two chunks into their slots, then q_c at the tokens of c's
  // younger siblings that fall in these chunks (read by the walk, after this kernel)
  auto publish = [&](int c, double Lq) {
    double s0 = 0.0, s1 = 0.0;
#pragma unroll
    for (int e = 0; e < E2; ++e)
      if (vidx(e) < V) {
        if (e < EPT) s0 += rb[e];
        else s1 += rb[e];
      }
    s0 = wave_sum_f64(s0);
    s1 = wave_sum_f64(s1);
    if ((tid & 63) == 0) {
      red[0][tid >> 6] = s0;
      red[1][tid >> 6] = s1;
    }
    __syncthreads();
    if (tid < 2 && 2 * pair + tid < nz) {
      double t = 0.0;
#pragma unroll
      for (int q = 0; q < kThreads / kWave; ++q) t += red[tid][q];
      __hip_atomic_store(reinterpret_cast<uint64_t*>(p.zpart) +
                             (static_cast<size_t>(b) * K + c) * nz + 2 * pair + tid,
                         static_cast<uint64_t>(__double_as_longlong(t)), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid < K && ((p.younger[c] >> tid) & 1u)) {
      const int xs = tok_sh[tid];
      if (xs >= base && xs < min(base + 2 * kZChunk, V))
        p.qpair[(static_cast<size_t>(b) * K + tid) * kMaxBlock + c] =
            exp(static_cast<double>(logit_at<kBF16>(p.draft, qrow_of(c) + xs)) * it - Lq);
    }
  };
  // q of the pass after next is loaded at the top of a pass and exponentiated after the
  // publish, off the path from one pass's sums to the next pass's
  auto load_q = [&](int c) { load_row(xq, p.draft, qrow_of(c)); };
  if (m > 2) load_q(p.child_list[cs + 1]);
  publish(p.child_list[cs], ln_sh[1]);
  if (m > 2) {
#pragma unroll
    for (int e = 0; e < E2; ++e) {
      qv[e] = exp(static_cast<double>(xq[e]) * it - ln_sh[2]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const double Lp = ln_sh[0];
  for (int j = 2; j < m; ++j) {
    const int c = p.child_list[cs + j - 1], cp = p.child_list[cs + j - 2];
    if (j + 1 < m) load_q(p.child_list[cs + j]);
    if (tid < kWave) {                              // Z_{j-1}, once every slot is written
      const uint64_t* z = reinterpret_cast<const uint64_t*>(p.zpart) +
                          (static_cast<size_t>(b) * K + cp) * nz;
      double sz = 0.0;
      for (int tries = 0;; ++tries) {
        bool empty = false;
        sz = 0.0;
        // a poll has its loads in flight together, one per slot (lanes past the last
        // slot load nothing); each lane sums its slots in increasing order
        for (int q0 = 0; q0 < nz; q0 += kPollLoads * kWave) {
          uint64_t bits[kPollLoads];
#pragma unroll
          for (int k = 0; k < kPollLoads; ++k) {
            const int q = q0 + k * kWave + tid;
            bits[k] = q < nz ? __hip_atomic_load(z + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                             : 0;
          }
#pragma unroll
          for (int k = 0; k < kPollLoads; ++k)
            if (q0 + k * kWave + tid < nz) {
              empty |= bits[k] == kSlotEmpty;
              sz += __longlong_as_double(static_cast<long long>(bits[k]));
            }
        }
        if (__ballot(empty) == 0) break;
        if (tries >= p.wait_limit) {                  // reported through the outputs
          if (tid == 0) p.fail[b] = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      sz = wave_sum_f64(sz);
      if (tid == 0) {
        zprev_sh = sz;
        if (pair == 0) p.ztab[static_cast<size_t>(b) * K + cp] = sz;
      }
    }
    __syncthreads();
    const double zp = zprev_sh;
    if (!(zp > 0.0)) {                              // Z_{j-1} = 0: the residual restarts at p_u
#pragma unroll
      for (int e = 0; e < E2; ++e) {
        const float xp = logit_at<kBF16>(p.target, trow + min(vidx(e), V - 1));
        rb[e] = fmax(0.0, exp(static_cast<double>(xp) * it - Lp) - qv[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < E2; ++e) rb[e] = fmax(0.0, rb[e] / zp - qv[e]);
    }
    publish(c, ln_sh[j]);
    if (j + 1 < m) {
#pragma unroll
      for (int e = 0; e < E2; ++e) {
        qv[e] = exp(static_cast<double>(xq[e]) * it - ln_sh[j + 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E2; ++e)
    if (vidx(e) < V) buf[vidx(e)] = rb[e];
}

// ---- 3. the tests and the walk, one workgroup per sequence.  The other waves first
// gather everything the tests need, all loads in flight together: the row normalisers
// (from the first pass's table, or folded from the parts when no pass ran), the Z of
// every elder sibling (from the passes' table, or folded here for each branching node's
// second-to-last child, which no later pass folded) and each node's elder siblings'
// probabilities of its token (written by the passes).  Wave 0 meanwhile loads its own
// node's two logits and computes what needs none of that; then it decides every test
// (lane = node) and walks.
template <bool kBF16>
__global__ void __launch_bounds__(kWalkThreads)
tree_walk_kernel(const TreeSampleParams p) {
  __shared__ double lsh[2 * kMaxBlock];            // L: target row u at u, draft row of c at K-1+c
  __shared__ double zc[kMaxBlock];                 // Z after child c, from the passes' table
  __shared__ double zlast[kMaxBlock];              // Z after child c, folded here
  __shared__ double qv[kMaxBlock][kMaxBlock];      // [c][l]: q_l(x_c), elder sibling l's probability of c's token
  __shared__ int32_t nd_m[kMaxBlock], nd_last[kMaxBlock], nd_second[kMaxBlock], nd_slot[kMaxBlock];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int lane = tid & 63;
  const int b = blockIdx.x;
  const int K = p.K, V = p.V;
  const int32_t* tok_b = p.tokens + static_cast<size_t>(b) * (K - 1);
  if (wave > 0) {                                  // each wave meets exactly one barrier
    if (wave < 8) {
      // elder siblings' probabilities of each node's token (q_l(x_c), written by the pass
      // that subtracted l): wave w takes nodes c = w, w + 7, ..., lane l sibling l
      constexpr int kSlots = (kMaxBlock + 6) / 7;
      double v[kSlots];
#pragma unroll
      for (int sl = 0; sl < kSlots; ++sl) {
        const int c = min(wave + 7 * sl, K - 1);
        const bool mine = wave + 7 * sl < K && ((p.elder[c] >> lane) & 1u);
        v[sl] = mine ? p.qpair[(static_cast<size_t>(b) * K + c) * kMaxBlock + lane] : 0.0;
      }
#pragma unroll
      for (int sl = 0; sl < kSlots; ++sl) {
        const int c = wave + 7 * sl;
        if (c < K && ((p.elder[c] >> lane) & 1u)) qv[c][lane] = v[sl];
      }
    } else if (wave < 10) {
      // row normalisers and the passes' Z table, one thread per entry
      const int r = tid - 8 * kWave;               // 0 .. 127
      if (r < 2 * K - 1) {
        const int rho = r < K ? target_rho(b, K, r) : draft_rho(p.B, b, K, r - K + 1);
        lsh[r] = p.has_lnorm ? p.lnorm[rho] : fold_lnorm(p, rho);   // written by the first pass
      }
      if (r < K) zc[r] = p.ztab[static_cast<size_t>(b) * K + r];
      // every node's stop-record fields (child count, last and second-to-last child,
      // residual slot), so that the record needs no global load after the walk
      if (r < K) {
        const int m = p.child_count[r];
        const int cs = p.child_start[r];
        nd_m[r] = m;
        nd_last[r] = m > 0 ? p.child_list[cs + m - 1] : 1;
        nd_second[r] = m > 1 ? p.child_list[cs + m - 2] : 0;
        nd_slot[r] = p.branch_slot[r];
      }
    } else {
      // Z after each branching node's second-to-last child: the six waves' 16-lane groups
      // fold entries g, g + 24, ... of last_z, every partial of a round in flight
      constexpr int kGroups = (kWalkThreads / kWave - 10) * 4;
      constexpr int kU = 12;
      const int g = (wave - 10) * 4 + (lane >> 4), l16 = lane & 15;
      for (int k0 = 0; k0 < p.n_last; k0 += kGroups) {
        const int k = k0 + g;
        const int cz = p.last_z[min(k, p.n_last - 1)];
        const double* z = p.zpart + (static_cast<size_t>(b) * K + cz) * p.nz;
        double sz = 0.0;
        for (int q0 = l16; q0 < p.nz; q0 += 16 * kU) {
          double t[kU];
#pragma unroll
          for (int i = 0; i < kU; ++i) t[i] = q0 + 16 * i < p.nz ? z[q0 + 16 * i] : 0.0;
#pragma unroll
          for (int i = 0; i < kU; ++i) sz += t[i];
        }
        sz = group_sum_f64<4>(sz);
        if (l16 == 0 && k < p.n_last) zlast[cz] = sz;
      }
    }
    __syncthreads();
    return;
  }
  const double it = p.inv_t;
  const int c = lane + 1;                          // the draft node this lane tests
  const bool node = c < K;
  const int u = node ? p.parent[c] : 0;
  const bool first_child = node && p.elder[c] == 0;   // tested against p_u itself
  const int32_t x = node ? tok_b[c - 1] : -1;
  const bool in_v = x >= 0 && x < V;
  const int xs = in_v ? x : 0;
  const double lp = logit_at<kBF16>(p.target, (static_cast<size_t>(b) * K + u) * V + xs);
  const double lq = logit_at<kBF16>(p.draft, (static_cast<size_t>(b) * (K - 1) + (node ? c - 1 : 0)) * V + xs);
  const int rho_u = target_rho(b, K, u), rho_c = draft_rho(p.B, b, K, node ? c : 1);
  const double Lu = p.has_lnorm ? p.lnorm[rho_u] : fold_lnorm(p, rho_u);
  const double Lc = p.has_lnorm ? p.lnorm[rho_c] : fold_lnorm(p, rho_c);
  // everything that needs no gathered value, before the barrier: the uniform, a first
  // child's threshold, p_u and q_c at the token
  const U64x4 wv = philox(p.offset, static_cast<uint64_t>(b), static_cast<uint64_t>(c), 0, p.seed, 0);
  const double uc = to_uniform(wv.x[0]);
  const bool live = node && in_v && lp != -INFINITY;
  double thr = 0.0, pv = 0.0, qc = 0.0;
  if (live) {
    if (first_child) {                             // against p_u: the chain's log form
      thr = exp(fmin(0.0, (lp - lq) * it - (Lu - Lc)));
    } else {
      pv = exp(lp * it - Lu);
      qc = exp(lq * it - Lc);
    }
  }
  __syncthreads();                                 // the gathered values are in LDS
  if (live && !first_child) {
    double r = pv;
    // the elder siblings in increasing node order (the order they are tested in)
    for (uint64_t e = p.elder[c]; e; e &= e - 1) {
      const int ci = __builtin_ctzll(e);
      const double raw = fmax(0.0, r - qv[c][ci]);
      // Z after child ci: from the pass after it, or (a second-to-last child) folded here
      const double z = ((p.zl_mask >> ci) & 1u) ? zlast[ci] : zc[ci];
      r = z > 0.0 ? raw / z : pv;
    }
    thr = r == 0.0 ? 0.0 : (qc == 0.0 ? 1.0 : fmin(1.0, r / qc));
  }
  const bool pass = live && uc < thr;
  // the walk: at the current node the lowest-numbered passing child (children are
  // tested in increasing node order); node numbers only grow, so it ends within K-1 steps
  const int par = node ? u : -1;
  int cur = 0, a = 0;
  int32_t my_path = lane == 0 ? 0 : -1;            // lane j ends up holding path[j]
  for (int step = 1; step < K; ++step) {
    const uint64_t hit = __ballot(node && pass && par == cur);
    if (!hit) break;
    cur = __builtin_ctzll(hit) + 1;
    a = step;
    if (lane == step) my_path = cur;
  }
  const int32_t tok = node ? x : 0;
  const int32_t next_node = __shfl(my_path, lane < 63 ? lane + 1 : 63);   // path[j+1]
  const int32_t next_tok = __shfl(tok, next_node > 0 ? next_node - 1 : 0);
  if (lane < K) {
    const size_t o = static_cast<size_t>(b) * K + lane;
    if (lane != a) p.out_tokens[o] = lane < a ? next_tok : -1;   // slot a: the drawn token
    p.path[o] = my_path;
  }
  if (lane == 0) {
    // the race draws from max(0, rhat_{m-1} - q_c) at the stop node (every child c_1 ..
    // c_m rejected; c = c_m), or from p_u at a leaf
    const int m = nd_m[cur];
    TreeStop st;
    st.u = cur;
    st.m = m;
    st.c = nd_last[cur];
    st.slot = nd_slot[cur];
    st.zp = m > 1 ? zlast[nd_second[cur]] : 1.0;
    st.lp = lsh[cur];
    st.lq = m > 0 ? lsh[K - 1 + st.c] : 0.0;
    p.stop[b] = st;
    p.accept_len[b] = a;
  }
}

// ---- 4. the race over the stop node's last residual
template <bool kBF16>
__global__ void __launch_bounds__(kRaceThreads)
tree_race_kernel(const TreeSampleParams p) {
  __shared__ double rk[2][kRaceThreads / kWave];
  __shared__ int32_t ri[2][kRaceThreads / kWave];
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x;
  const int b = blockIdx.y;
  const int K = p.K, V = p.V;
  const double it = p.inv_t;
  const TreeStop st = p.stop[b];
  const int u = st.u, m = st.m, c = st.c;
  const double zp = st.zp;
  const bool from_buf = m > 1 && zp > 0.0;         // rhat_{m-1} from the stored residual
  const double* buf = p.resid + (static_cast<size_t>(b) * p.nbranch + st.slot) * V;
  const size_t trow = (static_cast<size_t>(b) * K + u) * V;
  const size_t qrow = (static_cast<size_t>(b) * (K - 1) + (c - 1)) * V;
  const int jb = chunk * p.race_chunk + 4 * tid;   // one Philox block (4 tokens) a thread
  double bk_r = INFINITY, bk_p = INFINITY;
  int32_t bi_r = 0x7FFFFFFF, bi_p = 0x7FFFFFFF;
  // every element load is issued before any is used (clamped, in-bounds indices; the
  // draft row is valid whatever m is, c being 1 at a leaf; the stored residual only
  // under the workgroup-uniform from_buf): a load inside the element loop made the
  // compiler wait for each in turn, three round trips per element
  float xp[4], xq[4];
  double rb[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int v = min(jb + e, V - 1);
    xp[e] = logit_at<kBF16>(p.target, trow + v);
    xq[e] = logit_at<kBF16>(p.draft, qrow + v);
  }
  if (from_buf) {
#pragma unroll
    for (int e = 0; e < 4; ++e) rb[e] = buf[min(jb + e, V - 1)];
  }
  if (jb < V) {
    const U64x4 w = philox(p.offset, static_cast<uint64_t>(b), kResample | static_cast<uint64_t>(u),
                           static_cast<uint64_t>(jb >> 2), p.seed, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = jb + e;
      if (v >= V) break;
      const double pv = exp(static_cast<double>(xp[e]) * it - st.lp);
      double r = pv;
      if (m > 0) {
        const double rh = from_buf ? rb[e] / zp : pv;
        const double qv = exp(static_cast<double>(xq[e]) * it - st.lq);
        r = fmax(0.0, rh - qv);
      }
      const double ej = neg_log1m(to_uniform(w.x[e]));
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
  block_best<kRaceThreads>(bk_r, bi_r, bk_p, bi_p, rk, ri);
  uint64_t* const keys = reinterpret_cast<uint64_t*>(p.race_key);
  if (tid == 0) {
    const size_t slot = (static_cast<size_t>(b) * p.race_nchunk + chunk) * 2;
    __hip_atomic_store(keys + slot, static_cast<uint64_t>(__double_as_longlong(bk_r)),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p.race_idx + slot, bi_r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(keys + slot + 1, static_cast<uint64_t>(__double_as_longlong(bk_p)),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p.race_idx + slot + 1, bi_p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (chunk != static_cast<int>(gridDim.x) - 1) return;

  // ---- the sequence's last chunk: the winner over every chunk, then the drawn token.
  // Every other chunk of the sequence has a lower workgroup id, so in-order dispatch has
  // started it before this one, and none of them waits on anything: each thread polls
  // its chunk's slot until it is written (the (key, index) minimum is order-independent).
  __syncthreads();                                 // rk, ri are reused
  const int a = p.accept_len[b];                  // the walk's, before this launch
  const int failed = p.fail[b];                   // a residual pass's wait gave up
  double fk_r = INFINITY, fk_p = INFINITY;
  int32_t fi_r = 0x7FFFFFFF, fi_p = 0x7FFFFFFF;
  bool gave_up = false;
  for (int q = tid; q < static_cast<int>(gridDim.x); q += kRaceThreads) {
    const size_t slot = (static_cast<size_t>(b) * p.race_nchunk + q) * 2;
    uint64_t k0, k1;
    int32_t i0, i1;
    for (int tries = 0;; ++tries) {
      k0 = __hip_atomic_load(keys + slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      k1 = __hip_atomic_load(keys + slot + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      i0 = __hip_atomic_load(p.race_idx + slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      i1 = __hip_atomic_load(p.race_idx + slot + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (k0 != kSlotEmpty && k1 != kSlotEmpty && i0 != kIdxEmpty && i1 != kIdxEmpty) break;
      if (tries >= p.wait_limit) {
        gave_up = true;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    const double d0 = __longlong_as_double(static_cast<long long>(k0));
    const double d1 = __longlong_as_double(static_cast<long long>(k1));
    if (better(d0, i0, fk_r, fi_r)) { fk_r = d0; fi_r = i0; }
    if (better(d1, i1, fk_p, fi_p)) { fk_p = d1; fi_p = i1; }
  }
  // a thread whose wait gave up enters the key -inf with index kGaveUp, which wins the
  // minimum (every real key is >= 0), so the workgroup learns of it with no extra barrier
  if (gave_up) { fk_r = -INFINITY; fi_r = kGaveUp; }
  block_best<kRaceThreads>(fk_r, fi_r, fk_p, fi_p, rk, ri);
  gave_up = fk_r == -INFINITY && fi_r == kGaveUp;
  if (failed || gave_up) {                         // a wait gave up: the sequence reports -1
    if (tid < p.K) {
      p.out_tokens[static_cast<size_t>(b) * p.K + tid] = -1;
      p.path[static_cast<size_t>(b) * p.K + tid] = -1;
    }
    if (tid == 0) p.accept_len[b] = -1;
  } else if (tid == 0) {
    const int32_t token = (fk_r < INFINITY) ? fi_r : (fk_p < INFINITY ? fi_p : -1);
    p.out_tokens[static_cast<size_t>(b) * p.K + a] = token;
  }
}

}  // namespace

// Workspace, in order: zpart [B][K][nz], resid [B][K/2][V] (fp64), race_key
// [B][race_nchunk][2], part_s [B(2K-1)][kNormSplit], lnorm [B(2K-1)], qpair [B][K][64],
// ztab [B][K], stop [B] records,
// race_idx [B][race_nchunk][2], part_m [B(2K-1)][kNormSplit] (fp32).
size_t sample_tree_workspace_bytes(int B, int K, int V) {
  const size_t rows = static_cast<size_t>(B) * (2 * K - 1);
  const size_t nz = (static_cast<size_t>(V) + kZChunk - 1) / kZChunk;
  const size_t nrace = (static_cast<size_t>(V) + kRaceChunk - 1) / kRaceChunk;
  size_t off = 0;
  off += static_cast<size_t>(B) * K * nz * sizeof(double);      // zpart
  off += static_cast<size_t>(B) * (K / 2) * V * sizeof(double); // resid: at most K/2 branching nodes
  off += static_cast<size_t>(B) * nrace * 2 * sizeof(double);   // race_key
  off += rows * kNormSplit * sizeof(double);                    // part_s
  off += rows * sizeof(double);                                 // lnorm
  off += static_cast<size_t>(B) * K * kMaxBlock * sizeof(double); // qpair
  off += static_cast<size_t>(B) * K * sizeof(double);           // ztab
  off += static_cast<size_t>(B) * sizeof(TreeStop);             // stop
  off += static_cast<size_t>(B) * nrace * 2 * sizeof(int32_t);  // race_idx
  off += rows * kNormSplit * sizeof(float);                     // part_m
  off += static_cast<size_t>(B) * sizeof(int32_t);              // fail
  return (off + 15) & ~static_cast<size_t>(15);
}

void carve_sample_tree_workspace(TreeSampleParams& p, void* workspace) {
  const size_t rows = static_cast<size_t>(p.B) * (2 * p.K - 1);
  char* w = static_cast<char*>(workspace);
  p.zpart = reinterpret_cast<double*>(w);
  w += static_cast<size_t>(p.B) * p.K * p.nz * sizeof(double);
  p.resid = reinterpret_cast<double*>(w);
  w += static_cast<size_t>(p.B) * (p.K / 2) * p.V * sizeof(double);
  p.race_key = reinterpret_cast<double*>(w);
  w += static_cast<size_t>(p.B) * p.race_nchunk * 2 * sizeof(double);
  p.part_s = reinterpret_cast<double*>(w);
  w += rows * kNormSplit * sizeof(double);
  p.lnorm = reinterpret_cast<double*>(w);
  w += rows * sizeof(double);
  p.qpair = reinterpret_cast<double*>(w);
  w += static_cast<size_t>(p.B) * p.K * kMaxBlock * sizeof(double);
  p.ztab = reinterpret_cast<double*>(w);
  w += static_cast<size_t>(p.B) * p.K * sizeof(double);
  p.stop = reinterpret_cast<TreeStop*>(w);
  w += static_cast<size_t>(p.B) * sizeof(TreeStop);
  p.race_idx = reinterpret_cast<int32_t*>(w);
  w += static_cast<size_t>(p.B) * p.race_nchunk * 2 * sizeof(int32_t);
  p.part_m = reinterpret_cast<float*>(w);
  w += rows * kNormSplit * sizeof(float);
  p.fail = reinterpret_cast<int32_t*>(w);
}

int plan_sample_tree(TreeSampleParams& p, const int32_t* parents_host, TreePassPlan& plan) {
  const int K = p.K;
  p.nz = (p.V + kZChunk - 1) / kZChunk;
  p.race_chunk = kRaceChunk;
  p.race_nchunk = (p.V + kRaceChunk - 1) / kRaceChunk;
  for (int i = 0; i < kMaxBlock; ++i) {
    p.parent[i] = -1;
    p.child_start[i] = 0;
    p.child_count[i] = 0;
    p.child_list[i] = 0;
    p.branch_slot[i] = 0;
    p.pass_node[i] = 0;
    p.last_z[i] = 0;
    p.elder[i] = 0;
  }
  int count[kMaxBlock] = {0};
  for (int i = 1; i < K; ++i) {
    const int par = parents_host[i - 1];
    p.parent[i] = static_cast<int8_t>(par);
    ++count[par];
  }
  int pos = 0;
  for (int u = 0; u < K; ++u) {
    p.child_start[u] = static_cast<int8_t>(pos);
    p.child_count[u] = static_cast<int8_t>(count[u]);
    for (int i = u + 1; i < K; ++i)
      if (parents_host[i - 1] == u) p.child_list[pos++] = static_cast<int8_t>(i);
  }
  for (int c = 1; c < K; ++c) {                    // elder siblings: same parent, lower number
    uint64_t e = 0;
    for (int i = 1; i < c; ++i)
      if (parents_host[i - 1] == parents_host[c - 1]) e |= 1ull << i;
    p.elder[c] = e;
  }
  for (int c = 0; c < kMaxBlock; ++c) p.younger[c] = 0;
  for (int c = 1; c < K; ++c)
    for (uint64_t e = p.elder[c]; e; e &= e - 1) p.younger[__builtin_ctzll(e)] |= 1ull << c;
  int nbr = 0, mmax = 0;
  p.n_last = 0;
  p.zl_mask = 0;
  for (int u = 0; u < K; ++u) {
    mmax = count[u] > mmax ? count[u] : mmax;
    if (count[u] > 1) {
      p.branch_slot[u] = static_cast<int8_t>(nbr++);
      p.last_z[p.n_last++] = p.child_list[p.child_start[u] + count[u] - 2];
      p.zl_mask |= 1ull << p.child_list[p.child_start[u] + count[u] - 2];
    }
  }
  p.nbranch = nbr > 0 ? nbr : 1;
  // pass j (1 .. mmax-1) covers the nodes with more than j children, by decreasing child
  // count (ties: node order); each gets a word (u, c_j, c_{j-1}, residual row)
  const int rounds = mmax > 1 ? mmax - 1 : 0;
  p.has_lnorm = rounds > 0 ? 1 : 0;               // the first pass writes the table
  int words = 0;
  for (int j = 1; j <= rounds; ++j) {
    plan.off[j] = words;
    for (int cnt = K - 1; cnt > j; --cnt)
      for (int u = 0; u < K; ++u) {
        if (count[u] != cnt) continue;
        const int c = p.child_list[p.child_start[u] + j - 1];
        const int cp = j > 1 ? p.child_list[p.child_start[u] + j - 2] : 0xFF;
        p.pass_node[words++] = u | (c << 8) | (cp << 16) | (p.branch_slot[u] << 24);
      }
    plan.n[j] = words - plan.off[j];
  }
  return rounds;
}

// Workgroups of the fused residual passes that the current device holds at once: an
// occupancy query and the device's compute-unit count, once per device (0 when either
// query fails, which keeps the per-pass launches).
template <bool kBF16>
int chain_resident() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 0;
  }
  int r = cached[dev].load(std::memory_order_relaxed);
  if (r == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, tree_residual_chain_kernel<kBF16>,
                                                     kThreads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();                    // not a launch's error: clear it
      return 0;
    }
    r = per_cu > 0 && cus > 0 ? per_cu * cus : -1;
    cached[dev].store(r, std::memory_order_relaxed);
  }
  return r > 0 ? r : 0;
}

hipError_t launch_sample_tree(const TreeSampleParams& p, const TreePassPlan& plan, int rounds,
                              sv_dtype dtype, hipStream_t stream) {
  const bool bf = dtype == SV_BF16;
  const int rows = p.B * (2 * p.K - 1);
  if (bf)
    hipLaunchKernelGGL(tree_row_norm_kernel<true>, dim3(kNormSplit, rows), dim3(kNormThreads), 0,
                       stream, p.target, p.draft, p.B, p.K, p.V, p);
  else
    hipLaunchKernelGGL(tree_row_norm_kernel<false>, dim3(kNormSplit, rows), dim3(kNormThreads), 0,
                       stream, p.target, p.draft, p.B, p.K, p.V, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // every pass in one launch when the workgroups of the nodes with three or more
  // children (pass 2's nodes, first in its grid) fit the device at once
  const int waiting_wg = rounds >= 2 ? (p.nz + 1) / 2 * p.B * plan.n[2] : 0;
  const bool fused =
      rounds >= 2 && waiting_wg <= (bf ? chain_resident<true>() : chain_resident<false>());
  for (int j = 1; j <= (fused ? 0 : rounds); ++j) {
    const dim3 g(p.nz, p.B * plan.n[j]);
    if (bf)
      hipLaunchKernelGGL(tree_residual_kernel<true>, g, dim3(kThreads), 0, stream, j, plan.off[j],
                         plan.n[j], p);
    else
      hipLaunchKernelGGL(tree_residual_kernel<false>, g, dim3(kThreads), 0, stream, j, plan.off[j],
                         plan.n[j], p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (fused) {
    const dim3 g((p.nz + 1) / 2, p.B * plan.n[1]);
    if (bf)
      hipLaunchKernelGGL(tree_residual_chain_kernel<true>, g, dim3(kThreads), 0, stream,
                         plan.off[1], p);
    else
      hipLaunchKernelGGL(tree_residual_chain_kernel<false>, g, dim3(kThreads), 0, stream,
                         plan.off[1], p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (bf) hipLaunchKernelGGL(tree_walk_kernel<true>, dim3(p.B), dim3(kWalkThreads), 0, stream, p);
  else hipLaunchKernelGGL(tree_walk_kernel<false>, dim3(p.B), dim3(kWalkThreads), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 gr(p.race_nchunk, p.B);
  if (bf) hipLaunchKernelGGL(tree_race_kernel<true>, gr, dim3(kRaceThreads), 0, stream, p);
  else hipLaunchKernelGGL(tree_race_kernel<false>, gr, dim3(kRaceThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sv
