// Latent visual compressor (SpecFLASH README, "components", compressor equation):
//     out[b] = softmax(scale * C . F_b^T) . F_b,   softmax over the N feature rows.
//
// Pass 1 (scores_kernel): S_b = scale * C . F_b^T on MFMA 32x32x16 fp16.  Grid (N/64
// tile, b); four waves own 32x32 blocks of the 64 (queries) x 64 (features) tile and
// read both operands straight from global memory (each lane 16 contiguous bytes of a
// query row and of a feature row per step), fp32 scores to the workspace.
// Pass 2 (out_kernel): grid (D/128 tile, b).  The workgroup turns its C score rows into
// unnormalised fp16 weights exp(s - max) in LDS with fp32 row sums, then streams F_b in
// 32-row tiles, transposing each tile into LDS (the contraction runs over the feature
// rows, so the MFMA operand needs 8 consecutive rows of one column), and accumulates
// out = W . F_b / rowsum on MFMA.
#include "common.hpp"
#include "internal.hpp"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxN = 1024;
constexpr int kNT = 32;                 // feature rows per pass-2 tile
constexpr int kDT = 128;                // output columns per pass-2 workgroup

__global__ void __launch_bounds__(kThreads) scores_kernel(const CompressParams p) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wc = wave >> 1, wn = wave & 1;
  const int b = blockIdx.y;
  const int n0 = blockIdx.x * 64 + wn * 32;
  const int c = wc * 32 + l32;            // query row of the A operand
  const int n = n0 + l32;                 // feature row of the B operand
  const uint16_t* qrow = static_cast<const uint16_t*>(p.queries) + static_cast<size_t>(c) * p.D;
  const uint16_t* frow =
      static_cast<const uint16_t*>(p.feats) + (static_cast<size_t>(b) * p.N + n) * p.D;
  const bool qa = c < p.C, fa = n < p.N;
  if (wc * 32 >= p.C) return;            // no query rows for this wave
  f32x16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
  constexpr int U = 8;
  for (int d0 = 0; d0 < p.D; d0 += 16 * U) {
    u32x4 av[U], bv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int d = d0 + u * 16 + h * 8;
      av[u] = qa ? *reinterpret_cast<const u32x4*>(qrow + d) : u32x4{0u, 0u, 0u, 0u};
      bv[u] = fa ? *reinterpret_cast<const u32x4*>(frow + d) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc = Mfma<TagF16>::step(av[u], bv[u], acc);
  }
  if (!fa) return;
  float* srow = p.scores + static_cast<size_t>(b) * p.C * p.N + n;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int cc = wc * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
    if (cc < p.C) srow[static_cast<size_t>(cc) * p.N] = acc[r] * p.scale;
  }
}

__global__ void __launch_bounds__(kThreads) out_kernel(const CompressParams p) {
  constexpr int WROW = kMaxN + 8;                 // fp16 weight row (padded)
  constexpr int FROW = kNT + 8;                   // transposed feature tile row (padded)
  __shared__ __align__(16) uint16_t w_lds[64 * WROW];
  __shared__ __align__(16) uint16_t f_lds[kDT * FROW];
  __shared__ float rsum[64];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int b = blockIdx.y;
  const int dbase = blockIdx.x * kDT;
  const int N = p.N;
  const int Npad = (N + kNT - 1) / kNT * kNT;

  // ---- weights: wave w owns query rows w, w+4, ...
  for (int c = wave; c < 64; c += 4) {
    uint16_t* wr = &w_lds[c * WROW];
    if (c >= p.C) {
      for (int n = lane; n < Npad; n += 64) wr[n] = 0;
      if (lane == 0) rsum[c] = 1.0f;
      continue;
    }
    const float* srow = p.scores + (static_cast<size_t>(b) * p.C + c) * N;
    float m = -INFINITY;
    for (int n = lane; n < N; n += 64) m = fmaxf(m, srow[n]);
    m = wave_max(m);
    float sum = 0.0f;
    for (int n = lane; n < Npad; n += 64) {
      uint16_t wv = 0;
      if (n < N) {
        wv = f32_to_f16(__expf(srow[n] - m));
        sum += f16_to_f32(wv);
      }
      wr[n] = wv;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    if (lane == 0) rsum[c] = sum;
  }

  // ---- out tile: wave (wc, wd) owns query rows 32*wc.. and columns 64*wd.. (2 blocks)
  const int wc = wave >> 1, wd = wave & 1;
  const bool active = wc * 32 < p.C;
  f32x16 acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;

  // feature tile load: kNT rows x kDT columns = 512 chunks of 16 B, 2 per thread
  const uint16_t* fb = static_cast<const uint16_t*>(p.feats) + static_cast<size_t>(b) * N * p.D;
  for (int nt = 0; nt < Npad; nt += kNT) {
    u32x4 v[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int ch = tid + kThreads * u;
      const int r = ch >> 4;                      // feature row in the tile
      const int col = (ch & 15) * 8;              // first of 8 columns
      v[u] = (nt + r < N) ? *reinterpret_cast<const u32x4*>(fb + static_cast<size_t>(nt + r) * p.D + dbase + col)
                          : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();                              // previous tile fully consumed
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int ch = tid + kThreads * u;
      const int r = ch >> 4;
      const int col = (ch & 15) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        f_lds[(col + e) * FROW + r] = static_cast<uint16_t>(v[u][e >> 1] >> (16 * (e & 1)));
    }
    __syncthreads();
    if (active) {
#pragma unroll
      for (int ks = 0; ks < kNT / 16; ++ks) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&w_lds[(wc * 32 + l32) * WROW + nt + ks * 16 + h * 8]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4 bo = *reinterpret_cast<const u32x4*>(&f_lds[(wd * 64 + t * 32 + l32) * FROW + ks * 16 + h * 8]);
          acc[t] = Mfma<TagF16>::step(a, bo, acc[t]);
        }
      }
    }
  }
  if (!active) return;
  uint16_t* ob = static_cast<uint16_t*>(p.out) + static_cast<size_t>(b) * p.C * p.D;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = wc * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (c < p.C)
        ob[static_cast<size_t>(c) * p.D + dbase + wd * 64 + t * 32 + l32] = f32_to_f16(acc[t][r] / rsum[c]);
    }
}

}  // namespace

size_t compress_workspace_bytes(int B, int C, int N) {
  return static_cast<size_t>(B) * C * N * sizeof(float);
}

hipError_t launch_compress(const CompressParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(scores_kernel, dim3((p.N + 63) / 64, p.B), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(out_kernel, dim3(p.D / kDT, p.B), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sv
