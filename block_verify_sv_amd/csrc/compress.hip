// Latent visual compressor (SpecFLASH README, "components", compressor equation):
//     out[b] = softmax(scale * C . F_b^T) . F_b,   softmax over the N feature rows.
//
// Pass 1 (scores_kernel): C . F_b^T on MFMA 32x32x16 fp16, as two partial sums over
// the halves of d.  Grid (64-feature tile, b, half); both operands are staged through
// LDS in 64-d steps from coalesced loads held in a register ring.
// Pass 2 (softmax_kernel): one wave per query row adds the two partial sums, scales,
// and turns the scores into fp16 weights exp(s - max) and their fp32 sum (of the
// rounded weights).
// Pass 3 (out_kernel): grid (D/128 tile, b).  The workgroup streams F_b in 32-row tiles
// (with the 256-column tile, non-temporal loads: this is the features' last use in the
// call, while pass 1 reads them with ordinary loads so that this pass finds them in the
// Infinity Cache) through a register ring (several tiles in flight, each with its weight
// operands read from the cache-resident workspace) into LDS as loaded; the contraction
// runs over the feature rows, so each MFMA operand (8 consecutive rows of one column)
// comes from two LDS transpose reads.  out = W . F_b / rowsum accumulates on MFMA.
#include "common.hpp"
#include "internal.hpp"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxC = 64;
constexpr int kSK = 64;                 // pass-1 contraction step (d per LDS tile)
constexpr int kSRing = 4;               // pass-1 register ring (kSRing - 1 steps in flight)
constexpr int kNT = 32;                 // feature rows per pass-3 tile
constexpr int kRing = 3;                // pass-3 register ring (kRing - 1 tiles in flight)

__host__ __device__ __forceinline__ int pad_n(int N) { return (N + kNT - 1) / kNT * kNT; }

// Pass 1.  Workgroup (64-feature tile, image b, contraction half kh): the 64 x 64 score
// tile over d in [kh*D/2, (kh+1)*D/2), as the kh-th of two partial sums (the softmax
// pass adds them in order).  Both operands are staged in 64-d steps: coalesced 16-byte
// loads (8 lanes per 128-byte row segment) into a register ring kSRing-1 steps ahead,
// then padded LDS tiles that the four 32x32 MFMA blocks read.
// Kernels take the fields their first loads need as leading plain arguments (preloaded
// into SGPRs), then the whole parameter block.
__global__ void __launch_bounds__(kThreads)
scores_kernel(const void* queries, const void* feats, float* scores, int32_t B, int32_t C,
              int32_t N, int32_t D, const CompressParams p) {
  constexpr int ROW = kSK + 8;                     // LDS row: 64 d + 16 bytes of padding
  __shared__ __align__(16) uint16_t q_lds[2][64 * ROW];
  __shared__ __align__(16) uint16_t f_lds[2][64 * ROW];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wc = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * 64;
  const int b = blockIdx.y;
  const int kh = blockIdx.z;
  const bool active = wc * 32 < C;
  const int steps = (D >> 1) / kSK;
  const int dbeg = kh * (D >> 1);
  // load mapping: chunk ch = tid + 256u covers row ch/8, 8 halves at column 8*(ch%8);
  // rows past C (queries) or N (features) are clamped in bounds and never stored
  const uint16_t* qsrc[2];
  const uint16_t* fsrc[2];
  int loff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ch = tid + kThreads * u;
    const int r = ch >> 3, col = (ch & 7) * 8;
    qsrc[u] = static_cast<const uint16_t*>(queries) + static_cast<size_t>(min(r, C - 1)) * D + dbeg + col;
    fsrc[u] = static_cast<const uint16_t*>(feats) +
              (static_cast<size_t>(b) * N + min(n0 + r, N - 1)) * D + dbeg + col;
    loff[u] = r * ROW + col;
  }
  struct ST { u32x4 q[2], f[2]; };
  auto load = [&](ST& t, int st) {
    const int d = min(st, steps - 1) * kSK;       // past the end: re-read the last step
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      t.q[u] = *reinterpret_cast<const u32x4*>(qsrc[u] + d);
      t.f[u] = *reinterpret_cast<const u32x4*>(fsrc[u] + d);
    }
  };
  f32x16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
  auto step = [&](const ST& t, int st) {
    uint16_t* ql = q_lds[st & 1];
    uint16_t* fl = f_lds[st & 1];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      *reinterpret_cast<u32x4*>(&ql[loff[u]]) = t.q[u];
      *reinterpret_cast<u32x4*>(&fl[loff[u]]) = t.f[u];
    }
    __syncthreads();                               // step st in LDS; st-1's buffer free
    if (active && st < steps) {
#pragma unroll
      for (int ks = 0; ks < kSK / 16; ++ks) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&ql[(wc * 32 + l32) * ROW + ks * 16 + h * 8]);
        const u32x4 bo = *reinterpret_cast<const u32x4*>(&fl[(wn * 32 + l32) * ROW + ks * 16 + h * 8]);
        acc = Mfma<TagF16>::step(a, bo, acc);
      }
    }
  };
  ST ring[kSRing];
#pragma unroll
  // The prologue loads are kept in step order, and the loop runs whole groups of kSRing
  // steps (past the last step: loads re-read it, the MFMAs are skipped).  The compiler's
  // wait counts merge every path into the loop head: loads issued out of order, or an
  // exit from the middle of a group, would make them drain the ring once per group.
  for (int u = 0; u < kSRing - 1; ++u) {
    load(ring[u], u);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int s0 = 0; s0 < steps; s0 += kSRing) {
#pragma unroll
    for (int u = 0; u < kSRing; ++u) {
      const int st = s0 + u;
      load(ring[(u + kSRing - 1) % kSRing], st + kSRing - 1);
      step(ring[u], st);                         // past the last step: no MFMA
    }
  }
  const int n = n0 + wn * 32 + l32;
  if (!active || n >= N) return;
  float* srow = scores + (static_cast<size_t>(kh) * B + b) * C * N + n;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int cc = wc * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
    if (cc < C) srow[static_cast<size_t>(cc) * N] = acc[r];
  }
}

// One wave per query row (rows C..63 get zero weights and sum 1).
__global__ void __launch_bounds__(kThreads)
softmax_kernel(const float* scores, uint16_t* weights, float* rowsum, int32_t B, int32_t C,
               int32_t N, float scale, const CompressParams p) {
  constexpr int kPer = 1024 / 64;                  // scores per lane (N <= 1024)
  const int lane = threadIdx.x & 63;
  const int c = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  const int Nw = pad_n(N);
  uint16_t* wr = weights + (static_cast<size_t>(b) * kMaxC + c) * Nw;
  if (c >= C) {
    for (int n = lane; n < Nw; n += 64) wr[n] = 0;
    if (lane == 0) rowsum[b * kMaxC + c] = 1.0f;
    return;
  }
  const float* s0 = scores + (static_cast<size_t>(b) * C + c) * N;
  const float* s1 = s0 + static_cast<size_t>(B) * C * N;   // second contraction half
  float s[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {                 // all loads in flight
    const int n = min(lane + 64 * i, N - 1);
    s[i] = (s0[n] + s1[n]) * scale;
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (lane + 64 * i < N) m = fmaxf(m, s[i]);
  m = wave_max(m);
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int n = lane + 64 * i;
    if (n >= Nw) break;
    uint16_t wv = 0;
    if (n < N) {
      wv = f32_to_f16(__expf(s[i] - m));
      sum += f16_to_f32(wv);
    }
    wr[n] = wv;
  }
  sum = group_sum<6>(sum);
  if (lane == 0) rowsum[b * kMaxC + c] = sum;
}

// LDS transpose read (gfx950): within each 16-lane group, lane i receives 16-bit element
// i % 4 of the 8-byte rows addressed by lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(uint2, v);
}

// DT: output columns per workgroup, 256 for long feature streams when D allows (each
// wave then owns 4 column blocks of 32), else 128 (2 blocks).  The weight operand is read once per feature tile
// for all DT columns, so the wider tile halves the weight re-reads per feature byte.
template <int DT>
__global__ void __launch_bounds__(kThreads)
out_kernel(const void* feats, const uint16_t* weights, const float* rowsum, const float* scores,
           void* out, int32_t B, int32_t C, int32_t N, int32_t D, const CompressParams p) {
  // feature tile row: DT columns padded by 32 halves (DT + 32 halves = 16 banks mod 64),
  // so the four rows one half-wave's transpose read touches start 16 banks apart
  constexpr int FROW = DT + 32;
  constexpr int NB = DT / 64;                      // 32-column blocks per wave
  constexpr int CPR = DT / 8;                      // 16-byte chunks per tile row
  constexpr int CPT = kNT * CPR / kThreads;        // chunks per thread per tile
  static_assert(CPT * kThreads == kNT * CPR, "tile chunks per thread");
  __shared__ __align__(16) uint16_t f_lds[2][kNT * FROW];
  __shared__ float rsum[kMaxC];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int b = blockIdx.y;
  const int dbase = blockIdx.x * DT;
  const int Nw = pad_n(N);
  if (tid < kMaxC) rsum[tid] = rowsum[b * kMaxC + tid];

  // ---- out tile: wave (wc, wd) owns query rows 32*wc.. and columns (DT/2)*wd.. (NB
  // blocks).
  // The weight operand (8 consecutive feature rows of one query row per lane) comes
  // straight from the workspace (cache-resident: every d tile of the image reads it).
  const int wc = wave >> 1, wd = wave & 1;
  const bool active = wc * 32 < C;
  // transpose-read address of this lane: lane 4j + q of a 16-lane group points at row
  // 8h + j, columns 16*(group & 1) + 4q .. +3, so lane i of the group receives rows
  // 8h .. 8h+3 of column 16*(group & 1) + i: the MFMA B operand's layout
  const int grp = lane >> 4, i16 = lane & 15;
  const int tr_off = (h * 8 + (i16 >> 2)) * FROW + (grp & 1) * 16 + 4 * (i16 & 3);
  const uint16_t* wsrc = weights + (static_cast<size_t>(b) * kMaxC + wc * 32 + l32) * Nw + h * 8;
  f32x16 acc[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;

  // feature tiles: kNT rows x DT columns in chunks of 16 B, CPT per thread, held in a
  // register ring with the tile's weight operands; tile rows past N (the last tile)
  // re-read row N-1 and meet weights that are zero
  const uint16_t* fb = static_cast<const uint16_t*>(feats) + static_cast<size_t>(b) * N * D;
  const int nt_count = Nw / kNT;
  struct FT { u32x4 v[CPT]; u32x4 a[kNT / 16]; };
  auto load = [&](FT& f, int t) {
    const int nt = min(t, nt_count - 1) * kNT;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int ch = tid + kThreads * u;
      const int r = min(nt + ch / CPR, N - 1);
      const u32x4* src = reinterpret_cast<const u32x4*>(fb + static_cast<size_t>(r) * D + dbase + (ch % CPR) * 8);
      if constexpr (DT == 256)
        f.v[u] = __builtin_nontemporal_load(src);   // long streams: measured 82.0 -> 80.7 us
      else
        f.v[u] = *src;                             // (36, 324): ordinary loads measured faster
    }
#pragma unroll
    for (int ks = 0; ks < kNT / 16; ++ks) f.a[ks] = *reinterpret_cast<const u32x4*>(wsrc + nt + ks * 16);
  };
  auto tile = [&](const FT& f, int t) {
    uint16_t* fl = f_lds[t & 1];
#pragma unroll
    for (int u = 0; u < CPT; ++u) {                // row-major, as loaded
      const int ch = tid + kThreads * u;
      *reinterpret_cast<u32x4*>(&fl[(ch / CPR) * FROW + (ch % CPR) * 8]) = f.v[u];
    }
    __syncthreads();                               // tile t in LDS; tile t-1's buffer free
    if (active && t < nt_count) {
#pragma unroll
      for (int ks = 0; ks < kNT / 16; ++ks) {
#pragma unroll
        for (int tt = 0; tt < NB; ++tt) {
          // the operand (feature rows 16ks + 8h .. +7 of one column) as two transpose
          // reads of 4 rows each
          const uint16_t* src = &fl[ks * 16 * FROW + wd * (DT / 2) + tt * 32 + tr_off];
          const uint2 lo = lds_read_tr16(src);
          const uint2 hi = lds_read_tr16(src + 4 * FROW);
          const u32x4 bo = {lo.x, lo.y, hi.x, hi.y};
          acc[tt] = Mfma<TagF16>::step(f.a[ks], bo, acc[tt]);
        }
      }
    }
  };
  FT ring[kRing];
#pragma unroll
  for (int u = 0; u < kRing - 1; ++u) {          // in tile order; whole groups (as in pass 1)
    load(ring[u], u);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int t0 = 0; t0 < nt_count; t0 += kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      const int t = t0 + u;
      load(ring[(u + kRing - 1) % kRing], t + kRing - 1);
      tile(ring[u], t);                          // past the last tile: no MFMA
    }
  }
  if (!active) return;
  uint16_t* ob = static_cast<uint16_t*>(out) + static_cast<size_t>(b) * C * D;
#pragma unroll
  for (int t = 0; t < NB; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = wc * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (c < C)
        ob[static_cast<size_t>(c) * D + dbase + wd * (DT / 2) + t * 32 + l32] =
            f32_to_f16(acc[t][r] / rsum[c]);
    }
}

}  // namespace

size_t compress_workspace_bytes(int B, int C, int N) {
  const size_t scores = (2 * static_cast<size_t>(B) * C * N * sizeof(float) + 15) / 16 * 16;
  const size_t weights = static_cast<size_t>(B) * kMaxC * pad_n(N) * sizeof(uint16_t);
  return scores + weights + static_cast<size_t>(B) * kMaxC * sizeof(float);
}

void compress_bind_workspace(CompressParams& p, void* workspace) {
  char* w = static_cast<char*>(workspace);
  p.scores = reinterpret_cast<float*>(w);
  w += (2 * static_cast<size_t>(p.B) * p.C * p.N * sizeof(float) + 15) / 16 * 16;
  p.weights = reinterpret_cast<uint16_t*>(w);
  w += static_cast<size_t>(p.B) * kMaxC * pad_n(p.N) * sizeof(uint16_t);
  p.rowsum = reinterpret_cast<float*>(w);
}

hipError_t launch_compress(const CompressParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(scores_kernel, dim3((p.N + 63) / 64, p.B, 2), dim3(kThreads), 0, stream,
                     p.queries, p.feats, p.scores, p.B, p.C, p.N, p.D, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(softmax_kernel, dim3(kMaxC / (kThreads / 64), p.B), dim3(kThreads), 0, stream,
                     p.scores, p.weights, p.rowsum, p.B, p.C, p.N, p.scale, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the wide tile pays off on long feature streams (measured: N = 576 -6%, N = 324 +1%)
  if (p.D % 256 == 0 && p.N > 384)
    hipLaunchKernelGGL(out_kernel<256>, dim3(p.D / 256, p.B), dim3(kThreads), 0, stream,
                       p.feats, p.weights, p.rowsum, p.scores, p.out, p.B, p.C, p.N, p.D, p);
  else
    hipLaunchKernelGGL(out_kernel<128>, dim3(p.D / 128, p.B), dim3(kThreads), 0, stream,
                       p.feats, p.weights, p.rowsum, p.scores, p.out, p.B, p.C, p.N, p.D, p);
  return hipGetLastError();
}

}  // namespace sv
