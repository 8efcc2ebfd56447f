// Sampling acceptance: the standard speculative acceptance-rejection rule (SpecFLASH
// README, "components"), driven by counter-based Philox4x64-10 uniforms.
//
// Launch 1 (row_lse_kernel), grid (vocabulary chunk, row) over the B*K target rows and
// the B*(K-1) draft rows: per chunk the maximum m_c of the raw logits and
// s_c = sum exp((x - m_c) / T), fp32 exponentials accumulated in fp64.
//
// Launch 2 (sample_race_kernel), grid (vocabulary chunk, sequence): every workgroup
// combines the chunk partials into the row log-normalisers L = m/T + log sum_c s_c
// e^((m_c - m)/T) (fp64, fixed order), replays the K-1 ratio tests
//     lambda_k = (lp[k-1][d_k] - lq[k-1][d_k]) / T - (Lp_{k-1} - Lq_k),
//     accept d_k iff u_k < exp(min(0, lambda_k))            (fp64)
// to find the first rejection, then runs its chunk of the exponential race
//     key_j = -ln(1 - u_j) / r_j,  r = max(0, p_{k-1} - q_k) (or p_{K-1} for the bonus)
// in fp64, keeping the smallest key (lowest index on ties).  The last workgroup of a
// sequence reduces the chunk winners in chunk order and writes the outputs.  A race
// over p itself is carried along for the (measure-zero) case r == 0 everywhere.  The
// arrival counters are cleared by launch 1, so the workspace carries no state.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kLseThreads = 256;

// ---- Philox4x64-10 (Salmon et al., SC'11): multipliers and Weyl key increments of
// the 4x64 variant; ten rounds.
constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kPhiloxW1 = 0xBB67AE8584CAA73Bull;

struct U64x4 {
  uint64_t x[4];
};

__device__ __forceinline__ U64x4 philox(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                        uint64_t k0, uint64_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    const uint64_t hi0 = __umul64hi(kPhiloxM0, c0), lo0 = kPhiloxM0 * c0;
    const uint64_t hi1 = __umul64hi(kPhiloxM1, c2), lo1 = kPhiloxM1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return U64x4{{c0, c1, c2, c3}};
}

__device__ __forceinline__ double to_uniform(uint64_t w) {
  return static_cast<double>(w >> 11) * 0x1.0p-53;
}

template <bool kBF16>
__device__ __forceinline__ float logit_at(const void* base, size_t i) {
  if constexpr (kBF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
  else return static_cast<const float*>(base)[i];
}

// Row rho < B*K is target row rho; otherwise draft row rho - B*K.
template <bool kBF16>
__device__ __forceinline__ const void* row_ptr(const SampleParams& p, int rho) {
  const int nt = p.B * p.K;
  const size_t esz = kBF16 ? 2 : 4;
  if (rho < nt) return static_cast<const char*>(p.target) + static_cast<size_t>(rho) * p.V * esz;
  return static_cast<const char*>(p.draft) + static_cast<size_t>(rho - nt) * p.V * esz;
}

template <bool kBF16>
__global__ void __launch_bounds__(kLseThreads) row_lse_kernel(const SampleParams p) {
  __shared__ float redf[kLseThreads / kWave];
  __shared__ double redd[kLseThreads / kWave];
  const int tid = threadIdx.x;
  const int c = blockIdx.x;
  const int rho = blockIdx.y;
  // The race launch runs after this one on the same stream: clear its arrival counters
  // here, so the workspace needs no initial state whatever the previous call's shape.
  if (c == 0 && rho == 0)
    for (int i = tid; i < p.B; i += kLseThreads) p.counters[i] = 0u;
  const void* x = row_ptr<kBF16>(p, rho);
  const int j0 = c * p.chunk;
  const int j1 = min(j0 + p.chunk, p.V);
  constexpr int kMaxPer = 32;                      // chunk <= 8192 elements
  float v[kMaxPer];
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < kMaxPer; ++e) {
    const int j = j0 + tid + e * kLseThreads;
    v[e] = j < j1 ? logit_at<kBF16>(x, j) : -INFINITY;
    m = fmaxf(m, v[e]);
  }
  m = wave_max(m);
  if ((tid & 63) == 0) redf[tid >> 6] = m;
  __syncthreads();
  m = redf[0];
#pragma unroll
  for (int w = 1; w < kLseThreads / kWave; ++w) m = fmaxf(m, redf[w]);
  const float it = static_cast<float>(p.inv_t);
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < kMaxPer; ++e) s += static_cast<double>(expf((v[e] - m) * it));
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
}

struct Cand {
  double key;
  int32_t idx;
};
__device__ __forceinline__ bool better(double k, int32_t i, double bk, int32_t bi) {
  return k < bk || (k == bk && i < bi);
}

template <bool kBF16>
__global__ void __launch_bounds__(kThreads) sample_race_kernel(const SampleParams p) {
  __shared__ double Lrow[2 * kMaxBlock];
  __shared__ int32_t a_sh;
  __shared__ double rk[2][kThreads / kWave];
  __shared__ int32_t ri[2][kThreads / kWave];
  __shared__ bool is_last;

  const int tid = threadIdx.x;
  const int c = blockIdx.x;
  const int b = blockIdx.y;
  const int K = p.K;
  const double it = p.inv_t;

  // ---- row log-normalisers of this sequence: K target rows, then K-1 draft rows
  if (tid < 2 * K - 1) {
    const int rho = tid < K ? b * K + tid : p.B * K + b * (K - 1) + (tid - K);
    const float* pm = p.part_m + static_cast<size_t>(rho) * p.nchunk;
    const double* ps = p.part_s + static_cast<size_t>(rho) * p.nchunk;
    float m = -INFINITY;
    for (int q = 0; q < p.nchunk; ++q) m = fmaxf(m, pm[q]);
    double s = 0.0;
    for (int q = 0; q < p.nchunk; ++q)
      s += ps[q] * exp((static_cast<double>(pm[q]) - static_cast<double>(m)) * it);
    Lrow[tid] = static_cast<double>(m) * it + log(s);
  }
  __syncthreads();

  // ---- ratio tests in draft order; a = drafts accepted
  const int32_t* dr = p.drafts + static_cast<size_t>(b) * (K - 1);
  if (tid == 0) {
    int a = K - 1;
    for (int k = 1; k < K; ++k) {
      const int d = dr[k - 1];
      if (d < 0 || d >= p.V) {                    // a token outside the vocabulary is rejected
        a = k - 1;
        break;
      }
      const double lp = logit_at<kBF16>(p.target, (static_cast<size_t>(b) * K + k - 1) * p.V + d);
      const double lq = logit_at<kBF16>(p.draft, (static_cast<size_t>(b) * (K - 1) + k - 1) * p.V + d);
      const double lam = (lp - lq) * it - (Lrow[k - 1] - Lrow[K + k - 1]);
      const U64x4 w = philox(p.offset, static_cast<uint64_t>(b), static_cast<uint64_t>(k), 0,
                             p.seed, 0);
      const double u = to_uniform(w.x[0]);
      if (!(u < exp(fmin(0.0, lam)))) {
        a = k - 1;
        break;
      }
    }
    a_sh = a;
  }
  __syncthreads();
  const int a = a_sh;
  const bool resid = a < K - 1;
  const double Lp = Lrow[a];
  const double Lq = resid ? Lrow[K + a] : 0.0;
  const size_t prow = (static_cast<size_t>(b) * K + a) * p.V;
  const size_t qrow = (static_cast<size_t>(b) * (K - 1) + (resid ? a : 0)) * p.V;

  // ---- exponential race over this chunk (4 consecutive tokens per Philox block)
  const int j0 = c * p.chunk;
  const int j1 = min(j0 + p.chunk, p.V);
  double bk_r = INFINITY, bk_p = INFINITY;
  int32_t bi_r = 0x7FFFFFFF, bi_p = 0x7FFFFFFF;
  const uint64_t c2 = (1ull << 32) | static_cast<uint64_t>(a);
  for (int jb = j0 + 4 * tid; jb < j1; jb += 4 * kThreads) {
    const U64x4 w = philox(p.offset, static_cast<uint64_t>(b), c2, static_cast<uint64_t>(jb >> 2),
                           p.seed, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = jb + e;
      if (j >= j1) break;
      const double pj = exp(static_cast<double>(logit_at<kBF16>(p.target, prow + j)) * it - Lp);
      double rj = pj;
      if (resid) {
        const double qj = exp(static_cast<double>(logit_at<kBF16>(p.draft, qrow + j)) * it - Lq);
        rj = fmax(0.0, pj - qj);
      }
      const double ej = -log1p(-to_uniform(w.x[e]));
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
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double kr = __shfl_xor(bk_r, o);
    const int32_t ir = __shfl_xor(bi_r, o);
    if (better(kr, ir, bk_r, bi_r)) { bk_r = kr; bi_r = ir; }
    const double kp = __shfl_xor(bk_p, o);
    const int32_t ip = __shfl_xor(bi_p, o);
    if (better(kp, ip, bk_p, bi_p)) { bk_p = kp; bi_p = ip; }
  }
  if ((tid & 63) == 0) {
    rk[0][tid >> 6] = bk_r;
    ri[0][tid >> 6] = bi_r;
    rk[1][tid >> 6] = bk_p;
    ri[1][tid >> 6] = bi_p;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kThreads / kWave; ++w) {
      if (better(rk[0][w], ri[0][w], bk_r, bi_r)) { bk_r = rk[0][w]; bi_r = ri[0][w]; }
      if (better(rk[1][w], ri[1][w], bk_p, bi_p)) { bk_p = rk[1][w]; bi_p = ri[1][w]; }
    }
    const size_t slot = (static_cast<size_t>(b) * p.nchunk + c) * 2;
    p.race_key[slot] = bk_r;
    p.race_idx[slot] = bi_r;
    p.race_key[slot + 1] = bk_p;
    p.race_idx[slot + 1] = bi_p;
    __threadfence();
    const unsigned prev = atomicAdd(&p.counters[b], 1u);
    is_last = prev == static_cast<unsigned>(p.nchunk - 1);
  }
  __syncthreads();
  if (!is_last) return;

  // ---- last workgroup of sequence b: winner over chunks in chunk order
  __threadfence();
  if (tid == 0) {
    double kr = INFINITY, kp = INFINITY;
    int32_t ir = 0x7FFFFFFF, ip = 0x7FFFFFFF;
    for (int q = 0; q < p.nchunk; ++q) {
      const size_t slot = (static_cast<size_t>(b) * p.nchunk + q) * 2;
      const double k0 = __hip_atomic_load(&p.race_key[slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int32_t i0 = __hip_atomic_load(&p.race_idx[slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const double k1 = __hip_atomic_load(&p.race_key[slot + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int32_t i1 = __hip_atomic_load(&p.race_idx[slot + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (better(k0, i0, kr, ir)) { kr = k0; ir = i0; }
      if (better(k1, i1, kp, ip)) { kp = k1; ip = i1; }
    }
    const int32_t token = (kr < INFINITY) ? ir : ip;
    p.accept_len[b] = a;
    int32_t* out = p.out_tokens + static_cast<size_t>(b) * K;
    for (int i = 0; i < K; ++i) out[i] = i < a ? dr[i] : (i == a ? token : -1);
    __hip_atomic_store(&p.counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

int sample_chunk(int V) {
  (void)V;
  return 8192;
}

size_t sample_workspace_bytes(int B, int K, int V, int nchunk) {
  (void)V;
  const size_t rows = static_cast<size_t>(B) * (2 * K - 1);
  size_t off = 0;
  off += rows * nchunk * sizeof(double);          // part_s
  off += static_cast<size_t>(B) * nchunk * 2 * sizeof(double);  // race_key
  off += rows * nchunk * sizeof(float);           // part_m
  off += static_cast<size_t>(B) * nchunk * 2 * sizeof(int32_t); // race_idx
  off = (off + 15) & ~static_cast<size_t>(15);
  off += static_cast<size_t>(B) * sizeof(unsigned int);         // counters
  return off;
}

hipError_t launch_sample(const SampleParams& p, sv_dtype dtype, hipStream_t stream) {
  const dim3 g1(p.nchunk, p.B * (2 * p.K - 1));
  const dim3 g2(p.nchunk, p.B);
  if (dtype == SV_BF16) {
    hipLaunchKernelGGL(row_lse_kernel<true>, g1, dim3(kLseThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sample_race_kernel<true>, g2, dim3(kThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL(row_lse_kernel<false>, g1, dim3(kLseThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sample_race_kernel<false>, g2, dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace sv
