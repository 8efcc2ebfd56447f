// Block-verification attention for gfx950: split-KV pass + online-softmax merge pass.
//
// The target scores all K block rows in one forward over its whole context plus the
// block (VFlash-FM page, "How VFlash-FM works"): for each KV head g the K*G query rows
// of its head group form one dense (K*G) x d tile, so the scores S = Q_g K^T and the
// update O += P V are matrix products and run on MFMA (32x32x16 bf16/f16, 32x32x2 fp32).
//
// Split pass: one workgroup per (sequence b, KV head g, key split s).  Four waves; wave
// w owns query-row blocks w, w+4 (32 rows each).  Keys stream in tiles of 64 through
// LDS (double-buffered, the next tile's global loads in flight during the current
// tile's math).  Per tile and row block the wave computes S^T = K_tile . Q^T (keys on
// the MFMA M axis, query rows on N, so each lane owns one query row), applies the
// block mask, runs the online softmax in registers, and accumulates O^T = V^T . P^T.
// Output: unnormalised partial O, running max m (log2 units) and sum l per row.
//
// Merge pass: one wave per output row combines the splits in a fixed order:
//   m = max_s m_s, w_s = 2^(m_s - m), out = sum_s w_s O_s / sum_s w_s l_s,
//   lse = (m + log2 sum_s w_s l_s) * ln 2.
#include "common.hpp"
#include "internal.hpp"

namespace sv {
namespace {

constexpr int kTK = 64;           // keys per tile
constexpr int kThreads = 256;
constexpr float kNegBig = -1.0e30f;

// LDS row of key k within a tile: bits 2 and 3 swapped.  With this order the MFMA
// accumulator register r of lane-half h in a 32-key block holds key
// 16*(r/8) + 8*h + (r%8), so the P operand's 8 (16-bit) or 1 (fp32) consecutive
// registers cover consecutive keys and the V^T operand is one contiguous LDS read.
__device__ __forceinline__ int key_row(int k) {
  return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1);
}
__device__ __forceinline__ int key_of_reg(int r, int h) { return 16 * (r >> 3) + 8 * h + (r & 7); }

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// Zero the 16-bit elements e >= keep of a 16-byte chunk.
__device__ __forceinline__ u32x4 keep16(u32x4 v, int keep) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (2 * w >= keep) v[w] = 0u;
    else if (2 * w + 1 >= keep) v[w] &= 0xFFFFu;
  }
  return v;
}
// Zero the fp32 elements e >= keep of a 16-byte chunk.
__device__ __forceinline__ u32x4 keep32(u32x4 v, int keep) {
#pragma unroll
  for (int w = 0; w < 4; ++w)
    if (w >= keep) v[w] = 0u;
  return v;
}

template <class Tag, int D, int NRB>
__global__ void __launch_bounds__(kThreads, NRB == 1 ? 2 : 1) attn_split_kernel(const AttnParams p) {
  using S = typename Tag::store_t;
  using Op = typename Mfma<Tag>::op_t;
  constexpr int KPL = Tag::KPL;
  constexpr int SZ = Tag::kBytes;
  constexpr int EPC = 16 / SZ;                   // elements per 16-byte chunk
  constexpr int KROW = D + EPC;                  // K tile row (padded)
  constexpr int VROW = kTK + EPC;                // V^T tile row (padded)
  constexpr int CPK = D / EPC;                   // chunks per key row
  constexpr int K_PER_T = kTK * D / EPC / kThreads;
  constexpr int V_PER_T = D * kTK / EPC / kThreads;
  constexpr int KSTEPS = D / (2 * KPL);          // MFMA steps over d
  constexpr int PSTEPS = kTK / (2 * KPL);        // MFMA steps over the tile's keys
  constexpr int DB = D / 32;                     // 32-wide d blocks of O^T

  __shared__ __align__(16) S k_lds[2][kTK * KROW];
  __shared__ __align__(16) S v_lds[2][D * VROW];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int s = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;

  int ctx = p.ctx_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > p.max_ctx ? p.max_ctx : ctx);
  const int n_keys = ctx + p.K;
  const int k0 = s * p.chunk;
  if (k0 >= n_keys) return;                      // this sequence has fewer splits
  const int k1 = min(k0 + p.chunk, n_keys);
  const int Pm1 = (1 << p.P_log2) - 1;
  const int32_t* table = p.page_table + static_cast<size_t>(b) * p.max_pages;
  const S* kc = static_cast<const S*>(p.k_cache);
  const S* vc = static_cast<const S*>(p.v_cache);

  // ---- query operand (B of S^T = K . Q^T): lane owns query row 32*rb + l32
  Op qop[NRB][KSTEPS];
  uint64_t rmask[NRB];
  bool active[NRB];
#pragma unroll
  for (int t = 0; t < NRB; ++t) {
    const int rb = wave + 4 * t;
    const int r = rb * 32 + l32;
    active[t] = rb * 32 < p.R;
    rmask[t] = 0;
    const S* qp = nullptr;
    if (r < p.R) {
      const int i = r / p.G;
      const int head = g * p.G + (r - i * p.G);
      qp = static_cast<const S*>(p.q) + ((static_cast<size_t>(b) * p.K + i) * p.Hq + head) * D;
      rmask[t] = p.mask[i];
    }
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if constexpr (KPL == 8) {
        qop[t][ks] = qp ? *reinterpret_cast<const u32x4*>(qp + ks * 16 + h * 8) : zero4();
      } else {
        qop[t][ks] = qp ? static_cast<float>(qp[h * (D / 2) + ks]) : 0.0f;
      }
    }
  }

  // ---- tile staging: global -> registers -> LDS
  u32x4 kreg[K_PER_T];
  u32x4 vreg[V_PER_T];
  const int KR = min(Pm1 + 1, kTK);              // keys of one page inside a tile
  const int PPR = KR / EPC;                      // chunks per d row of such a run

  auto load_tile = [&](int kt) {
#pragma unroll
    for (int u = 0; u < K_PER_T; ++u) {
      const int c = tid + kThreads * u;
      const int key = c / CPK;
      const int part = c - key * CPK;
      const int pos = kt + key;
      u32x4 v = zero4();
      if (pos < k1) {
        const int page = table[pos >> p.P_log2];
        if (static_cast<unsigned>(page) < static_cast<unsigned>(p.num_pages)) {
          const size_t row = ((static_cast<size_t>(page) * p.Hkv + g) << p.P_log2) + (pos & Pm1);
          v = *reinterpret_cast<const u32x4*>(kc + row * D + part * EPC);
        }
      }
      kreg[u] = v;
    }
#pragma unroll
    for (int u = 0; u < V_PER_T; ++u) {
      const int c = tid + kThreads * u;
      const int run = c / (D * PPR);
      const int rem = c - run * D * PPR;
      const int d = rem / PPR;
      const int kg = run * PPR + (rem - d * PPR);  // EPC-key group inside the tile
      const int pos = kt + kg * EPC;
      u32x4 v = zero4();
      if (pos < k1) {
        const int page = table[pos >> p.P_log2];
        if (static_cast<unsigned>(page) < static_cast<unsigned>(p.num_pages)) {
          const size_t row = (static_cast<size_t>(page) * p.Hkv + g) * D + d;
          v = *reinterpret_cast<const u32x4*>(vc + (row << p.P_log2) + (pos & Pm1));
          if (pos + EPC > k1) v = (SZ == 2) ? keep16(v, k1 - pos) : keep32(v, k1 - pos);
        }
      }
      vreg[u] = v;
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < K_PER_T; ++u) {
      const int c = tid + kThreads * u;
      const int key = c / CPK;
      const int part = c - key * CPK;
      *reinterpret_cast<u32x4*>(&k_lds[buf][key_row(key) * KROW + part * EPC]) = kreg[u];
    }
#pragma unroll
    for (int u = 0; u < V_PER_T; ++u) {
      const int c = tid + kThreads * u;
      const int run = c / (D * PPR);
      const int rem = c - run * D * PPR;
      const int d = rem / PPR;
      const int kg = run * PPR + (rem - d * PPR);
      *reinterpret_cast<u32x4*>(&v_lds[buf][d * VROW + kg * EPC]) = vreg[u];
    }
  };

  // ---- running state
  float m_run[NRB], l_run[NRB];
  f32x16 oacc[NRB][DB];
#pragma unroll
  for (int t = 0; t < NRB; ++t) {
    m_run[t] = kNegBig;
    l_run[t] = 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[t][db][e] = 0.0f;
  }

  auto compute = [&](int buf, int kt) {
    const bool need_mask = (kt + kTK > ctx) || (kt + kTK > k1);
#pragma unroll
    for (int t = 0; t < NRB; ++t) {
      if (!active[t]) continue;
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.0f;
        const S* krow = &k_lds[buf][(kb * 32 + l32) * KROW];
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          Op a;
          if constexpr (KPL == 8) a = *reinterpret_cast<const u32x4*>(krow + ks * 16 + h * 8);
          else a = static_cast<float>(krow[h * (D / 2) + ks]);
          sacc[kb] = Mfma<Tag>::step(a, qop[t][ks], sacc[kb]);
        }
      }
      float sv[32];
      float mt = kNegBig;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sacc[kb][r] * p.scale_log2;
          if (need_mask) {
            const int pos = kt + kb * 32 + key_of_reg(r, h);
            bool vis = pos < k1;
            if (pos >= ctx) vis = vis && ((rmask[t] >> (pos - ctx)) & 1ull);
            x = vis ? x : -INFINITY;
          }
          sv[kb * 16 + r] = x;
          mt = fmaxf(mt, x);
        }
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run[t], mt);
      const float alpha = exp2f(m_run[t] - m_new);
      m_run[t] = m_new;
      float psum = 0.0f;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        sv[e] = exp2f(sv[e] - m_new);
        psum += sv[e];
      }
      l_run[t] = l_run[t] * alpha + psum;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[t][db][e] *= alpha;
#pragma unroll
      for (int ps = 0; ps < PSTEPS; ++ps) {
        Op bop;
        if constexpr (KPL == 8) {
          const float* pv = &sv[ps * 8];
          bop = u32x4{Tag::pack2(pv[0], pv[1]), Tag::pack2(pv[2], pv[3]),
                      Tag::pack2(pv[4], pv[5]), Tag::pack2(pv[6], pv[7])};
        } else {
          bop = sv[ps];
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const S* vrow = &v_lds[buf][(db * 32 + l32) * VROW];
          Op a;
          if constexpr (KPL == 8) {
            a = *reinterpret_cast<const u32x4*>(vrow + ps * 16 + h * 8);
          } else {
            a = static_cast<float>(vrow[32 * (ps >> 4) + key_of_reg(ps & 15, h)]);
          }
          oacc[t][db] = Mfma<Tag>::step(a, bop, oacc[t][db]);
        }
      }
    }
  };

  // ---- main loop: compute tile i from LDS while tile i+1 is fetched
  load_tile(k0);
  store_tile(0);
  __syncthreads();
  int buf = 0;
  for (int kt = k0; kt < k1; kt += kTK) {
    const bool more = kt + kTK < k1;
    if (more) load_tile(kt + kTK);
    compute(buf, kt);
    if (more) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // ---- partial results
#pragma unroll
  for (int t = 0; t < NRB; ++t) {
    if (!active[t]) continue;
    const float l_tot = l_run[t] + __shfl_xor(l_run[t], 32);
    const int r = (wave + 4 * t) * 32 + l32;
    if (r < p.R) {
      const size_t rowid = ((static_cast<size_t>(b) * p.Hkv + g) * p.nsplit + s) * p.R + r;
      float* po = p.part_o + rowid * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 v = {oacc[t][db][4 * q4 + 0], oacc[t][db][4 * q4 + 1],
                           oacc[t][db][4 * q4 + 2], oacc[t][db][4 * q4 + 3]};
          *reinterpret_cast<f32x4*>(po + db * 32 + q4 * 8 + h * 4) = v;
        }
      if (h == 0) p.part_ml[rowid] = make_float2(m_run[t], l_tot);
    }
  }
}

template <class Tag, int D>
__global__ void __launch_bounds__(kThreads) attn_merge_kernel(const AttnParams p) {
  using S = typename Tag::store_t;
  constexpr int EPL = D / 64;                    // output elements per lane
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;         // over B * K * Hq
  if (row >= p.B * p.K * p.Hq) return;
  const int hq = row % p.Hq;
  const int i = (row / p.Hq) % p.K;
  const int b = row / (p.Hq * p.K);
  const int g = hq / p.G;
  const int r = i * p.G + (hq - g * p.G);
  int ctx = p.ctx_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > p.max_ctx ? p.max_ctx : ctx);
  const int ns = (ctx + p.K + p.chunk - 1) / p.chunk;
  const size_t base = (static_cast<size_t>(b) * p.Hkv + g) * p.nsplit * p.R + r;

  float m = kNegBig;
  for (int s = lane; s < ns; s += 64) m = fmaxf(m, p.part_ml[base + static_cast<size_t>(s) * p.R].x);
  m = wave_max(m);
  float l = 0.0f;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
  for (int s = 0; s < ns; ++s) {
    const size_t id = base + static_cast<size_t>(s) * p.R;
    const float2 ml = p.part_ml[id];
    const float w = exp2f(ml.x - m);
    l += w * ml.y;
    const float* po = p.part_o + id * D;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += w * po[lane + 64 * e];
  }
  const float inv = 1.0f / l;
  S* out = static_cast<S*>(p.out) + ((static_cast<size_t>(b) * p.K + i) * p.Hq + hq) * D;
#pragma unroll
  for (int e = 0; e < EPL; ++e) out[lane + 64 * e] = Tag::from_f32(acc[e] * inv);
  if (p.lse && lane == 0)
    p.lse[(static_cast<size_t>(b) * p.K + i) * p.Hq + hq] = (m + log2f(l)) * 0.69314718055994531f;
}

template <class Tag, int D>
hipError_t launch_typed(const AttnParams& p, hipStream_t stream) {
  const dim3 grid(p.nsplit, p.Hkv, p.B);
  if ((p.R + 31) / 32 <= 4)
    hipLaunchKernelGGL((attn_split_kernel<Tag, D, 1>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_split_kernel<Tag, D, 2>), grid, dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = p.B * p.K * p.Hq;
  hipLaunchKernelGGL((attn_merge_kernel<Tag, D>), dim3((rows + 3) / 4), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnParams& p, int head_dim, sv_dtype dtype,
                            hipStream_t stream) {
  switch (dtype) {
    case SV_BF16:
      return head_dim == 128 ? launch_typed<TagBF16, 128>(p, stream)
                             : launch_typed<TagBF16, 64>(p, stream);
    case SV_F16:
      return head_dim == 128 ? launch_typed<TagF16, 128>(p, stream)
                             : launch_typed<TagF16, 64>(p, stream);
    case SV_F32:
      return head_dim == 128 ? launch_typed<TagF32, 128>(p, stream)
                             : launch_typed<TagF32, 64>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace sv
