// The target's LM head fused with greedy acceptance: logits = H . W^T for the block's
// hidden states H [M = B*K][Hd] against the output embedding W [V][Hd] (bf16 or fp16),
// reduced to each row's argmax without ever storing a logit, then the chain rule (the
// verify forward's last step before the acceptance of the VFlash-FM cycle figure).
//
// Pass 1 (lm_head_argmax_kernel): the vocabulary's 32-row units are shared out evenly
// over the workgroups, up to four each, one per wave as two 16-row MFMA blocks
// (16x16x32 bf16/f16, fp32 accumulate); the grid is sized to the chip's resident
// workgroups so that every CU streams about the same bytes.  The contraction
// runs over Hd in 32-column chunks, one MFMA each: lane (j, g) of a wave holds columns
// 32q + 8g .. 32q + 8g + 7 of W row v0 + 16*blk + j (and of H row j), loaded as 16 bytes
// straight into MFMA operand registers through a register ring; no LDS staging, no
// barriers in the loop.  The weight is read exactly once, so the pass is bound by HBM on
// it.  W comes either as the plain [V][Hd] matrix (each load instruction reads 64 bytes
// of 16 rows) or pre-packed by lm_head_pack_kernel into 1 KB tiles in exactly the order
// the waves consume them, so every load instruction of a wave reads one contiguous
// kilobyte; the packed stream is read with non-temporal loads.  The epilogue turns every
// logit into a packed key (orderable value bits << 32 | ~index), reduces each row over
// the wave's 32 columns with shuffles and over the four waves through LDS, and stores
// one key per (row, workgroup).
// Pass 2 (lm_head_finish_kernel): one workgroup per sequence folds each row's keys into
// its greedy token and walks the chain rule over them.
//
// Packed layout: W is cut into tiles of 16 rows x 32 columns.  Tile (u, q, h) covers rows
// 32u + 16h .. 32u + 16h + 15 and columns 32q .. 32q + 31; its 16-byte piece l = 16g + j
// holds row 32u + 16h + j, columns 32q + 8g .. 32q + 8g + 7 (the operand of lane l).
// Tiles are stored in the order u, then q, then h; rows at or past V are zero.  Size:
// ceil(V / 32) * 32 * Hd elements.
#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "internal.hpp"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kBlocks = 2;                        // 16-row MFMA blocks per wave
constexpr int kRowsPerWave = 16 * kBlocks;
constexpr int kSub = 2;                           // MFMA steps per load step (when Hd allows)
constexpr int kUnitsPerWG = kThreads / kWave;     // 32-row units per workgroup, at most
constexpr int kMaxResidentPerCU = 8;              // workgroups of four waves per CU, at most

typedef float f32x4v __attribute__((ext_vector_type(4)));

template <class Tag>
__device__ __forceinline__ f32x4v mfma16(u32x4 a, u32x4 b, f32x4v c);
template <>
__device__ __forceinline__ f32x4v mfma16<TagBF16>(u32x4 a, u32x4 b, f32x4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4v mfma16<TagF16>(u32x4 a, u32x4 b, f32x4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// MT = row tiles of 16 (M <= 16*MT).  The MFMA contraction pairs element e of lane
// (i, g) in A with element e of lane (j, g) in B, so any map of (g, e) to columns that
// both operands share sums every column exactly once; here lane (., g) holds columns
// 32q + 8g + e of chunk q in both.  One load step covers SUB chunks (MFMAs).
// PACKED: W is in the tile layout above (unit u = the wave's 32 rows).
// Kernels take the fields their first loads need as leading plain arguments (preloaded
// into SGPRs), then the whole parameter block.
template <class Tag, int MT, int SUB, int RING, bool PACKED>
__global__ void __launch_bounds__(kThreads)
lm_head_argmax_kernel(const void* hidden, const void* weight, int32_t M, int32_t V, int32_t Hd,
                      const LmHeadParams p) {
  static_assert(kBlocks == 2, "the packed tile order assumes 32-row units of two blocks");
  __shared__ uint64_t red[kThreads / kWave][16 * MT];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  // 32-row units shared out evenly: workgroup w takes units [w*U/nwg, (w+1)*U/nwg) (at
  // most four, one per wave); a wave without a unit loads nothing and keeps no key
  const int units = (V + kRowsPerWave - 1) / kRowsPerWave;
  const int ub = static_cast<int>(static_cast<int64_t>(blockIdx.x) * units / p.nwg);
  const int ue = static_cast<int>(static_cast<int64_t>(blockIdx.x + 1) * units / p.nwg);
  const int wv = __builtin_amdgcn_readfirstlane(wave);   // uniform: kept in scalar registers
  const bool live = ub + wv < ue;
  const int v0 = min(ub + wv, units - 1) * kRowsPerWave;
  const uint16_t* W = static_cast<const uint16_t*>(weight);
  const uint16_t* H = static_cast<const uint16_t*>(hidden);
  // rows past V or M are clamped in bounds; their keys are never kept
  const uint16_t* wrow[kBlocks];
  const u32x4* wunit = nullptr;
  if constexpr (PACKED) {
    wunit = reinterpret_cast<const u32x4*>(W + static_cast<size_t>(v0) * Hd) + lane;
  } else {
#pragma unroll
    for (int nb = 0; nb < kBlocks; ++nb)
      wrow[nb] = W + static_cast<size_t>(min(v0 + 16 * nb + l16, V - 1)) * Hd + 8 * g;
  }
  const uint16_t* hrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    hrow[mt] = H + static_cast<size_t>(min(16 * mt + l16, M - 1)) * Hd + 8 * g;

  const int steps = Hd / (32 * SUB);
  struct St { u32x4 w[kBlocks][SUB]; u32x4 h[MT][SUB]; };
  auto load = [&](St& s, int st) {
    const int q0 = min(st, steps - 1) * SUB;      // past the end: re-read the last step
#pragma unroll
    for (int nb = 0; nb < kBlocks; ++nb)
#pragma unroll
      for (int c = 0; c < SUB; ++c) {
        if constexpr (PACKED)
          s.w[nb][c] = __builtin_nontemporal_load(wunit + ((q0 + c) * kBlocks + nb) * kWave);
        else
          s.w[nb][c] = *reinterpret_cast<const u32x4*>(wrow[nb] + 32 * (q0 + c));
      }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int c = 0; c < SUB; ++c)
        s.h[mt][c] = *reinterpret_cast<const u32x4*>(hrow[mt] + 32 * (q0 + c));
  };
  f32x4v acc[MT][kBlocks];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nb = 0; nb < kBlocks; ++nb) acc[mt][nb] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};

  // The prologue loads are kept in step order and the loop runs whole groups of RING
  // steps (only the MFMAs are skipped past the end): the compiler merges the wait
  // counts of every path into the loop head, and a reordered prologue or an exit from
  // the middle of a group would make it drain the ring once per group.
  St ring[RING];
  if (live) {
#pragma unroll
  for (int u = 0; u < RING - 1; ++u) {
    load(ring[u], u);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int s0 = 0; s0 < steps; s0 += RING) {
#pragma unroll
    for (int u = 0; u < RING; ++u) {
      const int st = s0 + u;
      load(ring[(u + RING - 1) % RING], st + RING - 1);
      if (st < steps) {
#pragma unroll
        for (int c = 0; c < SUB; ++c)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nb = 0; nb < kBlocks; ++nb)
              acc[mt][nb] = mfma16<Tag>(ring[u].h[mt][c], ring[u].w[nb][c], acc[mt][nb]);
      }
    }
  }
  }

  // epilogue: lane (j, g) holds logit (row 16mt + 4g + r, column v0 + 16nb + j)
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint64_t best = 0;
#pragma unroll
      for (int nb = 0; nb < kBlocks; ++nb) {
        const int v = v0 + 16 * nb + l16;
        const uint64_t key = live && v < V ? argmax_key(acc[mt][nb][r], static_cast<uint32_t>(v)) : 0;
        best = key > best ? key : best;
      }
      best = group_max_u64<4>(best);               // over the 16 columns of the lane group
      if (l16 == 0) red[wave][16 * mt + 4 * g + r] = best;
    }
  }
  __syncthreads();
  if (tid < M) {
    uint64_t best = red[0][tid];
#pragma unroll
    for (int w = 1; w < kThreads / kWave; ++w) best = red[w][tid] > best ? red[w][tid] : best;
    p.part[static_cast<size_t>(tid) * p.nwg + blockIdx.x] = best;
  }
}

// One workgroup of 16 waves per sequence: wave w folds the per-workgroup keys of rows
// w, w + 16, ... of the sequence (20 loads per lane in flight, clamped indexes; a
// repeated key changes no maximum) into the row's greedy token, then wave 0 applies the
// chain rule to the K tokens: drafts are accepted while they equal the previous row's
// token, and the first row that disagrees (or the last row) gives the correction.
constexpr int kFinishThreads = 1024;
constexpr int kFinishLoads = 20;

__global__ void __launch_bounds__(kFinishThreads)
lm_head_finish_kernel(const unsigned long long* part, int32_t K, int32_t nwg,
                      const GreedyParams p) {
  __shared__ int32_t tok[64];
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the drafted token of lane k (draft k+1), loaded first (clamped, unconditional): it
  // shares the keys' round trip
  const int32_t dl = K > 1 ? p.drafts[static_cast<size_t>(b) * (K - 1) + min(lane, K - 2)] : 0;
  for (int r = wave; r < K; r += kFinishThreads / kWave) {
    const unsigned long long* src = part + (static_cast<size_t>(b) * K + r) * nwg;
    uint64_t best = 0;
    for (int base = 0; base < nwg; base += kFinishLoads * kWave) {
      uint64_t k[kFinishLoads];
#pragma unroll
      for (int u = 0; u < kFinishLoads; ++u) k[u] = src[min(base + u * kWave + lane, nwg - 1)];
#pragma unroll
      for (int u = 0; u < kFinishLoads; ++u) best = k[u] > best ? k[u] : best;
    }
    best = wave_max_u64(best);
    if (lane == 0) tok[r] = static_cast<int32_t>(argmax_key_index(best));
  }
  __syncthreads();
  if (wave != 0) return;
  const bool in = lane < K;
  const int32_t t = in ? tok[lane] : -1;
  // draft k+1 (drafts[b][k]) is checked against row k's token, k = 0 .. K-2
  const int32_t d = lane < K - 1 ? dl : 0;
  const uint64_t miss = __ballot(lane < K - 1 && d != t);
  const int a = miss ? __builtin_ctzll(miss) : K - 1;   // accepted drafts
  const int32_t corr = __shfl(t, a);
  if (in) {                                        // every store last
    if (p.argmax) p.argmax[static_cast<size_t>(b) * K + lane] = t;
    p.out_tokens[static_cast<size_t>(b) * K + lane] = lane < a ? d : (lane == a ? corr : -1);
  }
  if (lane == 0) p.accept_len[b] = a;
}

// Copies W [V][Hd] into the packed tile layout, one 16-byte piece per thread and step;
// pieces of rows at or past V are zero.
__global__ void __launch_bounds__(kThreads)
lm_head_pack_kernel(const u32x4* weight, u32x4* packed, int32_t V, int32_t Hd, int64_t pieces) {
  const int nq = Hd / 32;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < pieces;
       i += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int l = static_cast<int>(i & (kWave - 1));
    const int64_t tile = i / kWave;
    const int h = static_cast<int>(tile % kBlocks);
    const int64_t uq = tile / kBlocks;
    const int q = static_cast<int>(uq % nq);
    const int64_t row = (uq / nq) * kRowsPerWave + 16 * h + (l & 15);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < V) v = weight[row * (Hd / 8) + 4 * q + (l >> 4)];
    packed[i] = v;
  }
}

// Up to 16 rows with a 64-column-multiple width: two chunks per load step (128 contiguous
// bytes of a row, or 4 KB of the packed stream), 3-step ring (four waves per SIMD
// unpacked, five packed); otherwise single MFMA steps through a 6-step ring.
// Workgroups for the vocabulary's U units of 32 rows, given how many the chip keeps
// resident (a multiple of the CU count).  Units are shared out evenly over the grid, four
// per workgroup at most.  When the grid fits in one resident round it is rounded up to a
// whole number of workgroups per CU, so that every CU streams about U / 256 units
// (measured: 152,064 rows 167.9 -> 164.9 us, 100,000 rows 128.0 -> 118.5 us); a larger
// grid keeps four units per workgroup (whole resident rounds of fewer units measured
// slower).
int argmax_workgroups(int V, int resident) {
  const int units = (V + kRowsPerWave - 1) / kRowsPerWave;
  const int need = (units + kUnitsPerWG - 1) / kUnitsPerWG;
  if (need <= resident) return std::min(units, (need + kNumCUs - 1) / kNumCUs * kNumCUs);
  return need;
}

template <auto Kernel>
hipError_t launch_argmax(LmHeadParams& p, hipStream_t stream) {
  // workgroups resident on the chip: an occupancy query, once per kernel (a concurrent
  // first call only repeats the query)
  static std::atomic<int> cached{0};
  int resident = cached.load(std::memory_order_relaxed);
  if (resident == 0) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, Kernel, kThreads, 0) != hipSuccess) {
      (void)hipGetLastError();                    // not the launch's error: clear it
      per_cu = 1;
    }
    if (per_cu < 1) per_cu = 1;
    resident = std::min(per_cu, kMaxResidentPerCU) * kNumCUs;
    cached.store(resident, std::memory_order_relaxed);
  }
  p.nwg = argmax_workgroups(p.V, resident);
  hipLaunchKernelGGL(Kernel, dim3(p.nwg), dim3(kThreads), 0, stream, p.hidden, p.weight, p.M,
                     p.V, p.Hd, p);
  return hipGetLastError();
}

template <class Tag, bool PACKED>
hipError_t launch_typed(LmHeadParams& p, hipStream_t stream) {
  if (p.M <= 16 && p.Hd % (32 * kSub) == 0)
    return launch_argmax<lm_head_argmax_kernel<Tag, 1, kSub, 3, PACKED>>(p, stream);
  if (p.M <= 16) return launch_argmax<lm_head_argmax_kernel<Tag, 1, 1, 6, PACKED>>(p, stream);
  if (p.M <= 32) return launch_argmax<lm_head_argmax_kernel<Tag, 2, 1, 6, PACKED>>(p, stream);
  return launch_argmax<lm_head_argmax_kernel<Tag, 4, 1, 6, PACKED>>(p, stream);
}

}  // namespace

size_t lm_head_workspace_bytes(int M, int V) {
  // one key per (row, workgroup), for the largest grid argmax_workgroups can choose
  const int units = (V + kRowsPerWave - 1) / kRowsPerWave;
  const int most = std::max((units + kUnitsPerWG - 1) / kUnitsPerWG,
                            std::min(units, kMaxResidentPerCU * kNumCUs));
  return static_cast<size_t>(M) * most * sizeof(uint64_t);
}

size_t lm_head_packed_elems(int V, int Hd) {
  return static_cast<size_t>((V + kRowsPerWave - 1) / kRowsPerWave) * kRowsPerWave * Hd;
}

hipError_t launch_lm_head_pack(const void* weight, void* packed, int V, int Hd,
                               hipStream_t stream) {
  const int64_t pieces = static_cast<int64_t>(lm_head_packed_elems(V, Hd)) / 8;
  const int64_t blocks = std::min<int64_t>((pieces + kThreads - 1) / kThreads, 16384);
  hipLaunchKernelGGL(lm_head_pack_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                     0, stream, static_cast<const u32x4*>(weight), static_cast<u32x4*>(packed),
                     V, Hd, pieces);
  return hipGetLastError();
}

hipError_t launch_lm_head(const LmHeadParams& params, const GreedyParams& walk, sv_dtype dtype,
                          hipStream_t stream) {
  LmHeadParams p = params;                        // nwg is set by the argmax launch
  hipError_t e = p.packed
      ? (dtype == SV_F16 ? launch_typed<TagF16, true>(p, stream) : launch_typed<TagBF16, true>(p, stream))
      : (dtype == SV_F16 ? launch_typed<TagF16, false>(p, stream) : launch_typed<TagBF16, false>(p, stream));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lm_head_finish_kernel, dim3(walk.B), dim3(kFinishThreads), 0, stream,
                     p.part, walk.K, p.nwg, walk);
  return hipGetLastError();
}

}  // namespace sv
