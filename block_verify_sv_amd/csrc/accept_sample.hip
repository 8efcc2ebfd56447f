// Sampling acceptance: the standard speculative acceptance-rejection rule (SpecFLASH
// README, "components"), driven by counter-based Philox4x64-10 uniforms.
//
// Launch 1 (row_lse_kernel), grid (8192-entry vocabulary chunk, row) over the B*K
// target rows and the B*(K-1) draft rows: per chunk the maximum m_c of the raw logits
// and s_c = sum exp((x - m_c) / T), fp32 exponentials (the hardware exp2 unit)
// accumulated in fp64.  Logits may be -inf (probability 0, e.g. a masked vocabulary);
// a chunk of nothing but -inf contributes s_c = 0.
//
// Launch 2 (sample_race_kernel), grid (1024-entry vocabulary chunk, sequence).  Every
// workgroup combines the chunk partials into the row log-normalisers
//     L = m/T + log sum_c s_c e^((m_c - m)/T)            (fp64, fixed order),
// replays the K-1 ratio tests (one lane per draft, the first failure by ballot)
//     lambda_k = (lp[k-1][d_k] - lq[k-1][d_k]) / T - (Lp_{k-1} - Lq_k),
//     accept d_k iff u_k < exp(min(0, lambda_k))         (fp64),
// then runs its chunk of the exponential race
//     key_j = -ln(1 - u_j) / r_j,  r = max(0, p_{k-1} - q_k) (or p_{K-1} for the bonus)
// in fp64, one Philox block (4 tokens) per thread, keeping the smallest key (lowest
// index on ties); a race over p itself is carried along for the (measure-zero) case
// r == 0 everywhere.  Each chunk publishes its winners with agent-scope atomic stores
// into slots the first launch left empty (a signalling-NaN key, index -1); the last
// chunk workgroup of each sequence, started after every other one of its sequence by
// in-order dispatch, waits (bounded) until all its sequence's slots are written, reduces
// the winners and writes the outputs.  No fences or counters: each slot is its own
// ready flag, and the workspace carries no state between calls.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"
#include "sample_device.hpp"

namespace sv {
namespace {

constexpr int kThreads = 256;                     // race: 4 tokens per thread
constexpr int kLseThreads = 256;
constexpr int kLseChunk = 8192;                   // vocabulary entries per row_lse workgroup
constexpr int kRaceChunk = 4 * kThreads;          // vocabulary entries per race workgroup

// Row rho < nt = B*K is target row rho; otherwise draft row rho - B*K.
template <bool kBF16>
__device__ __forceinline__ const void* row_ptr(const void* target, const void* draft, int nt, int V,
                                               int rho) {
  const size_t esz = kBF16 ? 2 : 4;
  if (rho < nt) return static_cast<const char*>(target) + static_cast<size_t>(rho) * V * esz;
  return static_cast<const char*>(draft) + static_cast<size_t>(rho - nt) * V * esz;
}

// Each kernel takes the fields its first loads need as leading plain arguments
// (preloaded into SGPRs), then the whole parameter block.
template <bool kBF16>
__global__ void __launch_bounds__(kLseThreads)
row_lse_kernel(const void* target, const void* draft, int32_t B, int32_t K, int32_t V,
               int32_t chunk, const SampleParams p) {
  __shared__ float redf[kLseThreads / kWave];
  __shared__ double redd[kLseThreads / kWave];
  const int tid = threadIdx.x;
  const int c = blockIdx.x;
  const int rho = blockIdx.y;
  const void* x = row_ptr<kBF16>(target, draft, B * K, V, rho);
  const int j0 = c * chunk;
  const int j1 = min(j0 + chunk, V);
  constexpr int EPL = kBF16 ? 8 : 4;               // elements per 16-byte load
  constexpr int kLoads = kLseChunk / (kLseThreads * EPL);
  constexpr int kMaxPer = kLoads * EPL;
  float v[kMaxPer];
  if ((V % EPL) == 0) {
    // every load issued before any is consumed; clamped (in-bounds) indices past the
    // row end are masked afterwards
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int j = min(j0 + (tid + u * kLseThreads) * EPL, V - EPL);
      const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const char*>(x) +
                                                       static_cast<size_t>(j) * (kBF16 ? 2 : 4));
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        if constexpr (kBF16) v[u * EPL + e] = bf16_to_f32(static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1))));
        else v[u * EPL + e] = __uint_as_float(w[e]);
      }
    }
#pragma unroll
    for (int u = 0; u < kLoads; ++u)
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        if (j0 + (tid + u * kLseThreads) * EPL + e >= j1) v[u * EPL + e] = -INFINITY;
  } else {
#pragma unroll
    for (int e = 0; e < kMaxPer; ++e) {
      const int j = j0 + tid + e * kLseThreads;
      v[e] = logit_at<kBF16>(x, min(j, V - 1));
    }
#pragma unroll
    for (int e = 0; e < kMaxPer; ++e)
      if (j0 + tid + e * kLseThreads >= j1) v[e] = -INFINITY;
  }
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < kMaxPer; ++e) m = fmaxf(m, v[e]);
  m = wave_max(m);
  if ((tid & 63) == 0) redf[tid >> 6] = m;
  __syncthreads();
  m = redf[0];
#pragma unroll
  for (int w = 1; w < kLseThreads / kWave; ++w) m = fmaxf(m, redf[w]);
  // e^((x - m)/T) = 2^((x - m) * log2(e)/T) on the hardware exp unit.  A chunk whose
  // logits are all -inf (a masked stretch of the vocabulary) has m = -inf: subtracting 0
  // instead gives exp2(-inf) = 0 for every entry, so s = 0 and the chunk drops out of
  // the row's normaliser.
  const float it2 = static_cast<float>(p.inv_t * 1.4426950408889634);
  const float mref = m == -INFINITY ? 0.0f : m;
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < kMaxPer; ++e) s += static_cast<double>(fast_exp2((v[e] - mref) * it2));
  s = wave_sum_f64(s);
  if ((tid & 63) == 0) redd[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kLseThreads / kWave; ++w) t += redd[w];
    p.part_m[static_cast<size_t>(rho) * p.nchunk + c] = m;
    p.part_s[static_cast<size_t>(rho) * p.nchunk + c] = t;
  }
  // every race slot starts empty (each sequence's last race workgroup waits on them)
  const size_t slots = static_cast<size_t>(B) * p.race_nchunk * 2;
  const size_t stride = static_cast<size_t>(gridDim.x) * gridDim.y * kLseThreads;
  for (size_t i = (static_cast<size_t>(rho) * gridDim.x + c) * kLseThreads + tid; i < slots;
       i += stride) {
    reinterpret_cast<uint64_t*>(p.race_key)[i] = kSlotEmpty;
    p.race_idx[i] = kIdxEmpty;
  }
}

template <bool kBF16>
__global__ void __launch_bounds__(kThreads)
sample_race_kernel(const void* target, const void* draft, const int32_t* drafts, const float* part_m,
                   const double* part_s, int32_t B, int32_t K, int32_t V, int32_t nchunk,
                   const SampleParams p) {
  __shared__ double Lrow[2 * kMaxBlock];
  __shared__ int32_t a_sh;
  __shared__ double rk[2][kThreads / kWave];
  __shared__ int32_t ri[2][kThreads / kWave];

  const int tid = threadIdx.x;
  const int c = blockIdx.x;
  const int b = blockIdx.y;
  const double it = p.inv_t;
  const int32_t* dr = drafts + static_cast<size_t>(b) * (K - 1);

  // ---- start-up loads.  The drafted token of lane k-1 of wave 0 (which tests draft k)
  // comes first, then the chunk partials of the log-normalisers of the K target rows and
  // the K-1 draft rows (lpr lanes, a power of two aligned in the wave, share a row, each
  // taking every lpr-th partial, kFold of them per batch): all are issued before the first
  // wait.  Only the logits at the drafted tokens wait for a load (the token), and they
  // are issued before the partials are consumed, so the start-up costs two round trips.
  // Every index is clamped in bounds and every load is unconditional: a load under a
  // branch makes the compiler wait for it before the next one.
  const bool tester = tid < K - 1;
  const int32_t d = K > 1 ? dr[min(tid, K - 2)] : 0;
  const int nrows = 2 * K - 1;
  int lpr = 1;
  while (lpr * 2 * nrows <= kThreads && lpr < 16) lpr *= 2;
  const int row = tid / lpr, sub = tid - row * lpr;
  const bool has = row < nrows;
  const int rr = has ? row : 0;
  const int rho = rr < K ? b * K + rr : B * K + b * (K - 1) + (rr - K);
  const float* pm = part_m + static_cast<size_t>(rho) * nchunk;
  const double* ps = part_s + static_cast<size_t>(rho) * nchunk;
  constexpr int kFold = 8;
  float mv[kFold];
  double sv[kFold];
#pragma unroll
  for (int u = 0; u < kFold; ++u) {
    const int q = min(sub + u * lpr, nchunk - 1);
    mv[u] = pm[q];
    sv[u] = ps[q];
  }
  const bool in_vocab = d >= 0 && d < V;
  const int dc = in_vocab ? d : 0;
  const int tk = min(tid, K > 1 ? K - 2 : 0);
  const double lp = static_cast<double>(logit_at<kBF16>(target, (static_cast<size_t>(b) * K + tk) * V + dc));
  // at K = 1 there are no draft rows: the (unused) value is read from the target row
  const void* qsrc = K > 1 ? draft : target;
  const size_t qr = K > 1 ? static_cast<size_t>(b) * (K - 1) + tk : static_cast<size_t>(b) * K;
  const double lq = static_cast<double>(logit_at<kBF16>(qsrc, qr * V + dc));
  {
    // this lane's partials: q = sub, sub + lpr, ... in ascending order; the first batch is
    // already loaded, further batches (more than kFold * lpr chunks) are loaded in turn.
    // Maximum over the lane group, then every lane's sum against it, summed over the group
    // by shuffles (the same order whatever the batching).
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < kFold; ++u)
      if (sub + u * lpr < nchunk) m = fmaxf(m, mv[u]);
    for (int q = sub + kFold * lpr; q < nchunk; q += lpr) m = fmaxf(m, pm[q]);
    // over the lane group (lpr <= 16 lanes, aligned): uniform branches
    if (lpr > 1) m = fmaxf(m, xlane_f32<0>(m));
    if (lpr > 2) m = fmaxf(m, xlane_f32<1>(m));
    if (lpr > 4) m = fmaxf(m, xlane_f32<2>(m));
    if (lpr > 8) m = fmaxf(m, xlane_f32<3>(m));
    double s = 0.0;
#pragma unroll
    for (int u = 0; u < kFold; ++u)
      if (sub + u * lpr < nchunk)
        s += sv[u] * exp((static_cast<double>(mv[u]) - static_cast<double>(m)) * it);
    for (int q = sub + kFold * lpr; q < nchunk; q += lpr)
      s += ps[q] * exp((static_cast<double>(pm[q]) - static_cast<double>(m)) * it);
    if (lpr > 1) s += xlane_f64<0>(s);
    if (lpr > 2) s += xlane_f64<1>(s);
    if (lpr > 4) s += xlane_f64<2>(s);
    if (lpr > 8) s += xlane_f64<3>(s);
    if (has && sub == 0) Lrow[row] = static_cast<double>(m) * it + log(s);
  }
  __syncthreads();

  // ---- ratio tests, one lane per draft; a = drafts accepted = the first failure
  if (tid < 64) {
    bool fail = false;
    if (tester) {
      if (!in_vocab || lp == -INFINITY) {
        fail = true;     // a token outside the vocabulary, or one the target gives p = 0
      } else {           // q_k(d_k) = 0 < p: lambda = +inf, accepted
        const int k = tid + 1;
        const double lam = (lp - lq) * it - (Lrow[k - 1] - Lrow[K + k - 1]);
        const U64x4 w = philox(p.offset, static_cast<uint64_t>(b), static_cast<uint64_t>(k), 0,
                               p.seed, 0);
        fail = !(to_uniform(w.x[0]) < exp(fmin(0.0, lam)));
      }
    }
    const uint64_t fails = __ballot(fail);
    if (tid == 0) {
      const int a = fails ? __builtin_ctzll(fails) : K - 1;
      a_sh = a;
    }
  }
  __syncthreads();
  const int a = a_sh;
  const bool resid = a < K - 1;
  const double Lp = Lrow[a];
  const double Lq = resid ? Lrow[K + a] : 0.0;
  const size_t prow = (static_cast<size_t>(b) * K + a) * V;
  const size_t qrow = (static_cast<size_t>(b) * (K - 1) + (resid ? a : 0)) * V;

  // ---- exponential race over this chunk: one Philox block of 4 tokens per thread
  const int jb = c * p.race_chunk + 4 * tid;
  double bk_r = INFINITY, bk_p = INFINITY;
  int32_t bi_r = 0x7FFFFFFF, bi_p = 0x7FFFFFFF;
  if (jb < V) {
    float xp[4], xq[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {                 // clamped, in bounds; masked below
      const int j = min(jb + e, V - 1);
      xp[e] = logit_at<kBF16>(target, prow + j);
      xq[e] = logit_at<kBF16>(draft, qrow + j);
    }
    const uint64_t c2 = (1ull << 32) | static_cast<uint64_t>(a);
    const U64x4 w = philox(p.offset, static_cast<uint64_t>(b), c2, static_cast<uint64_t>(jb >> 2),
                           p.seed, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = jb + e;
      if (j >= V) break;
      const double pj = exp(static_cast<double>(xp[e]) * it - Lp);
      double rj = pj;
      if (resid) rj = fmax(0.0, pj - exp(static_cast<double>(xq[e]) * it - Lq));
      const double ej = neg_log1m(to_uniform(w.x[e]));
      if (rj > 0.0) {
        const double k = ej / rj;
        if (better(k, j, bk_r, bi_r)) { bk_r = k; bi_r = j; }
      }
      if (pj > 0.0) {
        const double k = ej / pj;
        if (better(k, j, bk_p, bi_p)) { bk_p = k; bi_p = j; }
      }
    }
  }
  block_best<kThreads>(bk_r, bi_r, bk_p, bi_p, rk, ri);
  uint64_t* const keys = reinterpret_cast<uint64_t*>(p.race_key);
  if (tid == 0) {
    const size_t slot = (static_cast<size_t>(b) * p.race_nchunk + c) * 2;
    __hip_atomic_store(keys + slot, static_cast<uint64_t>(__double_as_longlong(bk_r)),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p.race_idx + slot, bi_r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(keys + slot + 1, static_cast<uint64_t>(__double_as_longlong(bk_p)),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p.race_idx + slot + 1, bi_p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (c != static_cast<int>(gridDim.x) - 1) return;

  // ---- the sequence's last chunk: the winner over every chunk (the (key, index) minimum
  // is order-independent), then the outputs.  Every other chunk of the sequence has a
  // lower workgroup id, so in-order dispatch has started it before this one, and none of
  // them waits on anything: each thread polls its chunk's slot until it is written.
  __syncthreads();                                 // rk, ri are reused
  const int32_t dtok = K > 1 ? dr[min(tid, K - 2)] : 0;
  double fk_r = INFINITY, fk_p = INFINITY;
  int32_t fi_r = 0x7FFFFFFF, fi_p = 0x7FFFFFFF;
  bool gave_up = false;
  for (int q = tid; q < static_cast<int>(gridDim.x); q += kThreads) {
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
  block_best<kThreads>(fk_r, fi_r, fk_p, fi_p, rk, ri);
  gave_up = fk_r == -INFINITY && fi_r == kGaveUp;
  // a race with no positive weight (a row with no finite logit) draws nothing: -1; a
  // wait that gave up reports accept_len -1 and no tokens
  const int32_t token = (fk_r < INFINITY) ? fi_r : (fk_p < INFINITY ? fi_p : -1);
  if (tid < K)
    p.out_tokens[static_cast<size_t>(b) * K + tid] =
        gave_up ? -1 : (tid < a ? dtok : (tid == a ? token : -1));
  if (tid == 0) p.accept_len[b] = gave_up ? -1 : a;
}

}  // namespace

int sample_chunk(int V) {
  (void)V;
  return kLseChunk;
}

int sample_race_chunk(int V) {
  (void)V;
  return kRaceChunk;
}

size_t sample_workspace_bytes(int B, int K, int V) {
  const size_t rows = static_cast<size_t>(B) * (2 * K - 1);
  const size_t nchunk = (static_cast<size_t>(V) + kLseChunk - 1) / kLseChunk;
  const size_t nrace = (static_cast<size_t>(V) + kRaceChunk - 1) / kRaceChunk;
  size_t off = 0;
  off += rows * nchunk * sizeof(double);                    // part_s
  off += static_cast<size_t>(B) * nrace * 2 * sizeof(double);  // race_key
  off += rows * nchunk * sizeof(float);                     // part_m
  off += static_cast<size_t>(B) * nrace * 2 * sizeof(int32_t); // race_idx
  return (off + 15) & ~static_cast<size_t>(15);
}

hipError_t launch_sample(const SampleParams& p, sv_dtype dtype, hipStream_t stream) {
  const dim3 g1(p.nchunk, p.B * (2 * p.K - 1));
  const dim3 g2(p.race_nchunk, p.B);
#define LSE_ARGS p.target, p.draft, p.B, p.K, p.V, p.chunk, p
#define RACE_ARGS p.target, p.draft, p.drafts, p.part_m, p.part_s, p.B, p.K, p.V, p.nchunk, p
  if (dtype == SV_BF16) {
    hipLaunchKernelGGL(row_lse_kernel<true>, g1, dim3(kLseThreads), 0, stream, LSE_ARGS);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sample_race_kernel<true>, g2, dim3(kThreads), 0, stream, RACE_ARGS);
  } else {
    hipLaunchKernelGGL(row_lse_kernel<false>, g1, dim3(kLseThreads), 0, stream, LSE_ARGS);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sample_race_kernel<false>, g2, dim3(kThreads), 0, stream, RACE_ARGS);
  }
#undef LSE_ARGS
#undef RACE_ARGS
  return hipGetLastError();
}

}  // namespace sv
