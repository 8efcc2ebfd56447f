// Block-verification attention for gfx950: split-KV pass + online-softmax merge pass.
//
// The target scores all K block rows in one forward over its whole context plus the
// block (VFlash-FM page, "How VFlash-FM works"): for each KV head g the K*G query rows
// of its head group form one dense (K*G) x d tile, so the scores S = Q_g K^T and the
// update O += P V are matrix products and run on MFMA (32x32x16 bf16/f16, 32x32x2 fp32).
//
// Split pass: one workgroup per (sequence b, KV head g, key split s), sized so the
// grid is about one workgroup per compute unit.  Four waves; wave w owns query-row
// blocks w, w+4 (32 rows each).  The split's page ids are staged in LDS once, then keys
// stream in tiles of 64: a ring of four register tiles keeps three tiles (96 KB at bf16,
// d = 128) of global loads in flight while the fourth is written to one of two LDS
// buffers, so the HBM latency is covered without a dependent page-table load per tile.
// Per tile and row block the wave computes S^T = K_tile . Q^T (keys on the MFMA M axis,
// query rows on N, so each lane owns one query row), applies the block mask, runs the
// online softmax in registers, and accumulates O^T = V^T . P^T.
// Output per row: the partial output divided by its own sum, in the input dtype (half the
// bytes of fp32 for 16-bit inputs), its reference maximum m (log2 units) and sum l.
//
// Merge pass: one workgroup per output row; every (split, 32-element slice) pair has its
// own thread, so all partial loads are in flight at once, and the splits are combined
// in a fixed order:
//   m = max_s m_s, w_s = l_s 2^(m_s - m), out = sum_s w_s O_s / sum_s w_s,
//   lse = (m + log2 sum_s w_s) * ln 2      (O_s: split s's output, already divided by l_s).
#include "common.hpp"
#include "internal.hpp"

namespace sv {
namespace {

constexpr int kTK = 64;           // keys per tile
constexpr int kThreads = 256;     // merge pass
constexpr float kNegBig = -1.0e30f;
constexpr float kRescale = 8.0f;  // lazy-rescale threshold (log2 units)
#ifndef SV_RING_DEEP
#define SV_RING_DEEP 4
#endif
constexpr int kRingDeep = SV_RING_DEEP;
constexpr int kMaxSplitPages = kMaxSplitKeys / 16 + 2;

// LDS row of key k within a tile: bits 2 and 3 swapped.  With this order the MFMA
// accumulator register r of lane-half h in a 32-key block holds key
// 16*(r/8) + 8*h + (r%8), so the P operand's 8 (16-bit) or 1 (fp32) consecutive
// registers cover consecutive keys and the V^T operand is one contiguous LDS read.
__device__ __forceinline__ int key_row(int k) {
  return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1);
}
__device__ __forceinline__ int key_of_reg(int r, int h) { return 16 * (r >> 3) + 8 * h + (r & 7); }

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// Zero the 16-bit elements e >= keep of a 16-byte chunk (branch-free).
__device__ __forceinline__ u32x4 keep16(u32x4 v, int keep) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t m = (2 * w + 1 < keep) ? 0xFFFFFFFFu : ((2 * w < keep) ? 0xFFFFu : 0u);
    v[w] &= m;
  }
  return v;
}
// Zero the fp32 elements e >= keep of a 16-byte chunk (branch-free).
__device__ __forceinline__ u32x4 keep32(u32x4 v, int keep) {
#pragma unroll
  for (int w = 0; w < 4; ++w) v[w] &= (w < keep) ? 0xFFFFFFFFu : 0u;
  return v;
}

template <class Tag, int D, int NRB, int KW>
__global__ void __launch_bounds__(256 * KW, 1) attn_split_kernel(const AttnParams p) {
  using S = typename Tag::store_t;
  using Op = typename Mfma<Tag>::op_t;
  constexpr int T = 256 * KW;                    // threads: 4 row waves x KW key waves
  constexpr int KPL = Tag::KPL;
  constexpr int SZ = Tag::kBytes;
  constexpr int EPC = 16 / SZ;                   // elements per 16-byte chunk
  constexpr int KROW = D + EPC;                  // K tile row (padded)
  constexpr int VROW = kTK + EPC;                // V^T tile row (padded)
  constexpr int CPK = D / EPC;                   // chunks per key row
  constexpr int K_PER_T = kTK * D / EPC / T;
  constexpr int V_PER_T = D * kTK / EPC / T;
  constexpr int KSTEPS = D / (2 * KPL);          // MFMA steps over d
  constexpr int KBW = 2 / KW;                    // 32-key blocks per wave per tile
  constexpr int PSW = KBW * 32 / (2 * KPL);      // MFMA steps over one wave's keys
  constexpr int DB = D / 32;                     // 32-wide d blocks of O^T
  // register tiles in the load ring (RING-1 tiles in flight): deep for one row block
  // of 16-bit data, shallow where the row state already fills the register file
  constexpr int RING = (NRB == 1 && SZ == 2) ? kRingDeep : 2;
  constexpr int K_LDS = 2 * kTK * KROW * SZ;
  constexpr int V_LDS = 2 * D * VROW * SZ;
  static_assert(KW == 1 || NRB == 1, "key-split waves hold one row block each");
  static_assert(KW == 1 || 4 * 64 * (2 + DB * 16) * 4 <= K_LDS + V_LDS, "combine stage");

  __shared__ __align__(16) char smem[K_LDS + V_LDS];
  __shared__ int32_t pg_lds[kMaxSplitPages];
  S* const k_lds = reinterpret_cast<S*>(smem);
  S* const v_lds = reinterpret_cast<S*>(smem + K_LDS);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int rbw = wave & 3;                      // first row block of this wave
  const int kh = wave >> 2;                      // key half of each tile (KW == 2)
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

  // ---- page ids of this split, once (entries outside the pool become -1: read as zero)
  const int pg0 = k0 >> p.P_log2;
  const int npg = ((k1 - 1) >> p.P_log2) - pg0 + 1;
  for (int i = tid; i < npg; i += T) {
    const int pg = table[pg0 + i];
    pg_lds[i] = static_cast<unsigned>(pg) < static_cast<unsigned>(p.num_pages) ? pg : -1;
  }

  // ---- query operand (B of S^T = K . Q^T): lane owns query row 32*rb + l32
  Op qop[NRB][KSTEPS];
  uint64_t rmask[NRB];
  bool active[NRB];
#pragma unroll
  for (int t = 0; t < NRB; ++t) {
    const int rb = rbw + 4 * t;
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

  // ---- tile staging: global -> register ring -> LDS.  A 64-key tile is split into
  // runs of KR = min(P, 64) keys that lie in one page; each thread owns a fixed set of
  // 16-byte chunks (K_PER_T of K, V_PER_T of V) inside one run, so a tile costs one
  // page-id lookup per thread and constant offsets from two base pointers.  Loads are
  // branch-free: a run past the split end or on an unmapped page reads page 0 and is
  // zeroed when written to LDS -- never at load time, which would make the load wait
  // for its data and empty the ring.
  struct Tile {
    u32x4 k[K_PER_T];
    u32x4 v[V_PER_T];
    int ok;                                      // this thread's run is valid
  };
  const int KR = min(Pm1 + 1, kTK);              // keys of one run
  const int TPR = T * KR / kTK;                  // threads per run
  const int run = tid / TPR;
  const int li = tid - run * TPR;
  const int KGR = KR / EPC;                      // EPC-key groups per run row of V
  int k_goff[K_PER_T], k_loff[K_PER_T], v_goff[V_PER_T], v_loff[V_PER_T], v_key[V_PER_T];
#pragma unroll
  for (int u = 0; u < K_PER_T; ++u) {
    const int ci = li + TPR * u;
    const int key = ci / CPK, part = ci - (ci / CPK) * CPK;
    k_goff[u] = key * D + part * EPC;
    k_loff[u] = key_row(run * KR + key) * KROW + part * EPC;
  }
#pragma unroll
  for (int u = 0; u < V_PER_T; ++u) {
    const int ci = li + TPR * u;
    const int d = ci / KGR, kp = ci - (ci / KGR) * KGR;
    v_goff[u] = (d << p.P_log2) + kp * EPC;
    v_loff[u] = d * VROW + run * KR + kp * EPC;
    v_key[u] = run * KR + kp * EPC;              // first key of the chunk in the tile
  }

  // a page holds Hkv heads of P keys x D for K (token-major) and of D x P for V
  // (dim-major): the same element stride per page for both caches
  const uint32_t pstride = static_cast<uint32_t>(p.Hkv * D) << p.P_log2;
  const S* const kc_h = kc + (static_cast<size_t>(g * D) << p.P_log2);
  const S* const vc_h = vc + (static_cast<size_t>(g * D) << p.P_log2);
  auto load_tile = [&](Tile& r, int kt) {
    const int pos0 = kt + run * KR;
    const bool in = pos0 < k1;
    const int pg = pg_lds[in ? (pos0 >> p.P_log2) - pg0 : 0];
    r.ok = in && pg >= 0;
    const uint32_t page = r.ok ? static_cast<uint32_t>(pg) : 0u;
    const uint32_t slot = r.ok ? static_cast<uint32_t>(pos0 & Pm1) : 0u;
    const size_t poff = static_cast<size_t>(page) * pstride;   // one 32x32 -> 64-bit multiply
    const S* kb = kc_h + poff + slot * D;
    const S* vb = vc_h + poff + slot;
#pragma unroll
    for (int u = 0; u < K_PER_T; ++u) r.k[u] = *reinterpret_cast<const u32x4*>(kb + k_goff[u]);
#pragma unroll
    for (int u = 0; u < V_PER_T; ++u) r.v[u] = *reinterpret_cast<const u32x4*>(vb + v_goff[u]);
  };

  auto store_tile = [&](const Tile& r, int buf, int kt) {
    S* kl = k_lds + buf * kTK * KROW;
    S* vl = v_lds + buf * D * VROW;
    if (kt + kTK <= k1) {                        // interior tile: zero only unmapped runs
#pragma unroll
      for (int u = 0; u < K_PER_T; ++u)
        *reinterpret_cast<u32x4*>(kl + k_loff[u]) = r.ok ? r.k[u] : zero4();
#pragma unroll
      for (int u = 0; u < V_PER_T; ++u)
        *reinterpret_cast<u32x4*>(vl + v_loff[u]) = r.ok ? r.v[u] : zero4();
    } else {                                     // tail tile: also zero keys past k1
      const int left = k1 - kt;
#pragma unroll
      for (int u = 0; u < K_PER_T; ++u)
        *reinterpret_cast<u32x4*>(kl + k_loff[u]) = r.ok ? r.k[u] : zero4();
#pragma unroll
      for (int u = 0; u < V_PER_T; ++u) {
        u32x4 v = r.ok ? r.v[u] : zero4();
        v = (SZ == 2) ? keep16(v, left - v_key[u]) : keep32(v, left - v_key[u]);
        *reinterpret_cast<u32x4*>(vl + v_loff[u]) = v;
      }
    }
  };

  // ---- running state.  m_run is a reference maximum (raw score units) that only moves
  // when a row's maximum exceeds it by more than 2^kRescale in weight, so the O^T
  // accumulators are rescaled rarely; weights then stay below 2^kRescale.
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

  // Scores stay in raw dot-product units until the exponent: m_run and the row maxima
  // are raw maxima (scale > 0 keeps the order), and 2^(scale_log2 * (s - m)) is one fma
  // into the exp unit.
  const float c2 = p.scale_log2;
  const float resc = kRescale / c2;              // rescale threshold in raw units
  auto compute = [&](int buf, int kt) {
    const bool need_mask = (kt + kTK > ctx) || (kt + kTK > k1);
    const S* kbase = k_lds + buf * kTK * KROW;
    const S* vbase = v_lds + buf * D * VROW;
#pragma unroll
    for (int t = 0; t < NRB; ++t) {
      if (!active[t]) continue;
      float sv[16 * KBW];
#pragma unroll
      for (int kbi = 0; kbi < KBW; ++kbi) {
        const int kb = kh * KBW + kbi;
        const S* krow = kbase + (kb * 32 + l32) * KROW;
        Op kop[KSTEPS];
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          if constexpr (KPL == 8) kop[ks] = *reinterpret_cast<const u32x4*>(krow + ks * 16 + h * 8);
          else kop[ks] = static_cast<float>(krow[h * (D / 2) + ks]);
        }
        f32x16 acc;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) acc = Mfma<Tag>::step(kop[ks], qop[t][ks], acc);
        if (!need_mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sv[kbi * 16 + r] = acc[r];
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int pos = kt + kb * 32 + key_of_reg(r, h);
            const int t2 = pos - ctx;
            const bool vis = pos < k1 && (t2 < 0 || ((rmask[t] >> (t2 & 63)) & 1ull));
            sv[kbi * 16 + r] = vis ? acc[r] : -INFINITY;
          }
        }
      }
      float mt = sv[0];
#pragma unroll
      for (int e = 1; e < 16 * KBW; ++e) mt = fmaxf(mt, sv[e]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      if (__any(mt > m_run[t] + resc)) {         // wave-uniform: rare after the first tile
        const float m_new = fmaxf(m_run[t], mt);
        const float alpha = fast_exp2((m_run[t] - m_new) * c2);
        m_run[t] = m_new;
        l_run[t] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[t][db][e] *= alpha;
      }
      const float mneg = -m_run[t] * c2;
      float psum = 0.0f;
#pragma unroll
      for (int e = 0; e < 16 * KBW; ++e) {
        sv[e] = fast_exp2(fmaf(sv[e], c2, mneg));
        psum += sv[e];
      }
      l_run[t] += psum;
#pragma unroll
      for (int psi = 0; psi < PSW; ++psi) {
        const int ps = kh * PSW + psi;           // MFMA step within the tile
        Op bop;
        if constexpr (KPL == 8) {
          const float* pv = &sv[psi * 8];
          bop = u32x4{Tag::pack2(pv[0], pv[1]), Tag::pack2(pv[2], pv[3]),
                      Tag::pack2(pv[4], pv[5]), Tag::pack2(pv[6], pv[7])};
        } else {
          bop = sv[psi];
        }
        Op vop[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const S* vrow = vbase + (db * 32 + l32) * VROW;
          if constexpr (KPL == 8) {
            vop[db] = *reinterpret_cast<const u32x4*>(vrow + ps * 16 + h * 8);
          } else {
            vop[db] = static_cast<float>(vrow[32 * (ps >> 4) + key_of_reg(ps & 15, h)]);
          }
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[t][db] = Mfma<Tag>::step(vop[db], bop, oacc[t][db]);
      }
    }
  };

  // ---- main loop.  Tile j lives in ring slot j % RING and LDS buffer j % 2.  Step j
  // issues the loads of tile j+RING-1, computes tile j, then writes tile j+1 (loaded
  // RING-2 steps earlier) to the other LDS buffer; one barrier per step.  The ring loads
  // are issued unconditionally (past the last tile they re-read it, from cache): a load
  // under a branch makes the compiler's wait counts assume the path without it and
  // drain the whole ring before every LDS write.
  __syncthreads();                               // page ids visible
  const int nt = (k1 - k0 + kTK - 1) / kTK;
  auto tile_at = [&](int j) { return k0 + min(j, nt - 1) * kTK; };
  auto step = [&](int j, Tile& rl, const Tile& rs, int buf) {
    load_tile(rl, tile_at(j + RING - 1));
    compute(buf, k0 + j * kTK);
    if (j + 1 < nt) store_tile(rs, buf ^ 1, k0 + (j + 1) * kTK);
    __syncthreads();
  };
  Tile r[RING];
  load_tile(r[0], k0);
#pragma unroll
  for (int u = 1; u < RING - 1; ++u) load_tile(r[u], tile_at(u));
  store_tile(r[0], 0, k0);
  __syncthreads();
  for (int j0 = 0; j0 < nt; j0 += RING) {
#pragma unroll
    for (int u = 0; u < RING; ++u) {
      const int j = j0 + u;
      if (j >= nt) break;
      step(j, r[(u + RING - 1) % RING], r[(u + 1) % RING], j & 1);
    }
  }

  // ---- the row's sum over both lane halves, then (KW == 2) the two key-half waves of
  // a row block combine through LDS (the tile buffers are free after the last barrier)
#pragma unroll
  for (int t = 0; t < NRB; ++t) l_run[t] += __shfl_xor(l_run[t], 32);
  if constexpr (KW == 2) {
    constexpr int SW = 2 + DB * 16;              // floats staged per lane
    float* stage = reinterpret_cast<float*>(smem) + (rbw * 64 + lane) * SW;
    if (kh == 1 && active[0]) {
      stage[0] = m_run[0];
      stage[1] = l_run[0];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) stage[2 + db * 16 + e] = oacc[0][db][e];
    }
    __syncthreads();
    if (kh == 1) return;
    if (active[0]) {
      const float m2 = stage[0], l2 = stage[1];
      const float m = fmaxf(m_run[0], m2);
      const float a1 = fast_exp2((m_run[0] - m) * c2), a2 = fast_exp2((m2 - m) * c2);
      m_run[0] = m;
      l_run[0] = l_run[0] * a1 + l2 * a2;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[0][db][e] = oacc[0][db][e] * a1 + stage[2 + db * 16 + e] * a2;
    }
  }

  // ---- partial results: O / l in the input dtype, (m, l) in fp32
#pragma unroll
  for (int t = 0; t < NRB; ++t) {
    if (!active[t]) continue;
    const int r = (rbw + 4 * t) * 32 + l32;
    if (r < p.R) {
      const size_t rowid = ((static_cast<size_t>(b) * p.Hkv + g) * p.nsplit + s) * p.R + r;
      S* po = static_cast<S*>(p.part_o) + rowid * D;
      const float inv = l_run[t] > 0.0f ? 1.0f / l_run[t] : 0.0f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float o[4] = {oacc[t][db][4 * q4], oacc[t][db][4 * q4 + 1],
                              oacc[t][db][4 * q4 + 2], oacc[t][db][4 * q4 + 3]};
          S* dst = po + db * 32 + q4 * 8 + h * 4;
          if constexpr (SZ == 2) {
            const uint2 v = {Tag::pack2(o[0] * inv, o[1] * inv), Tag::pack2(o[2] * inv, o[3] * inv)};
            *reinterpret_cast<uint2*>(dst) = v;
          } else {
            *reinterpret_cast<f32x4*>(dst) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
          }
        }
      if (h == 0) p.part_ml[rowid] = make_float2(m_run[t] * c2, l_run[t]);   // m in log2 units
    }
  }
}

// 32 consecutive partial-output elements as floats.
template <class Tag>
__device__ __forceinline__ void load32(const typename Tag::store_t* src, float* x) {
  if constexpr (Tag::kBytes == 2) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(src + 8 * q);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        x[8 * q + e] = Tag::to_f32(static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1))));
    }
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const f32x4 w = *reinterpret_cast<const f32x4*>(src + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * q + e] = w[e];
    }
  }
}

template <class Tag, int D>
__global__ void __launch_bounds__(kThreads) attn_merge_kernel(const AttnParams p) {
  using S = typename Tag::store_t;
  constexpr int TPS = D / 32;                    // threads per split: 32 elements each
  constexpr int SPP = kThreads / TPS;            // splits per pass
  __shared__ float red[kThreads / kWave];
  __shared__ float acc_lds[SPP][D + 4];
  __shared__ float l_lds[SPP];

  const int tid = threadIdx.x;
  const int row = blockIdx.x;                    // over B * K * Hq
  const int hq = row % p.Hq;
  const int i = (row / p.Hq) % p.K;
  const int b = row / (p.Hq * p.K);
  const int g = hq / p.G;
  const int r = i * p.G + (hq - g * p.G);
  int ctx = p.ctx_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > p.max_ctx ? p.max_ctx : ctx);
  const int ns = (ctx + p.K + p.chunk - 1) / p.chunk;
  const size_t base = (static_cast<size_t>(b) * p.Hkv + g) * p.nsplit * p.R + r;
  const S* po = static_cast<const S*>(p.part_o);
  const int grp = tid / TPS;                     // split slot within a pass
  const int e0 = (tid % TPS) * 32;               // first element of this thread's slice

  // the first pass's partial slice goes in flight before the maximum is known
  float o[32];
  float ms = kNegBig, ls = 0.0f;
  if (grp < ns) {
    const size_t id = base + static_cast<size_t>(grp) * p.R;
    load32<Tag>(po + id * D + e0, o);
    const float2 ml = p.part_ml[id];
    ms = ml.x;
    ls = ml.y;
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) o[e] = 0.0f;
  }
  float m = ms;
  for (int s = grp + SPP; s < ns; s += SPP) m = fmaxf(m, p.part_ml[base + static_cast<size_t>(s) * p.R].x);
  m = wave_max(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / kWave; ++w) m = fmaxf(m, red[w]);

  const float w0 = grp < ns ? ls * fast_exp2(ms - m) : 0.0f;
  float lsum = w0;
#pragma unroll
  for (int e = 0; e < 32; ++e) o[e] *= w0;
  for (int s = grp + SPP; s < ns; s += SPP) {    // more splits than one pass holds
    const size_t id = base + static_cast<size_t>(s) * p.R;
    const float2 ml = p.part_ml[id];
    const float w = ml.y * fast_exp2(ml.x - m);
    lsum += w;
    float x[32];
    load32<Tag>(po + id * D + e0, x);
#pragma unroll
    for (int e = 0; e < 32; ++e) o[e] += w * x[e];
  }
#pragma unroll
  for (int q = 0; q < 8; ++q)
    *reinterpret_cast<f32x4*>(&acc_lds[grp][e0 + 4 * q]) = f32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
  if (tid % TPS == 0) l_lds[grp] = lsum;
  __syncthreads();

  const int nsp = ns < SPP ? ns : SPP;
  if (tid < D) {
    float a = 0.0f, l = 0.0f;
    for (int q = 0; q < nsp; ++q) {
      a += acc_lds[q][tid];
      l += l_lds[q];
    }
    S* out = static_cast<S*>(p.out) + ((static_cast<size_t>(b) * p.K + i) * p.Hq + hq) * D;
    out[tid] = Tag::from_f32(a / l);
    if (p.lse && tid == 0)
      p.lse[(static_cast<size_t>(b) * p.K + i) * p.Hq + hq] = (m + log2f(l)) * 0.69314718055994531f;
  }
}

template <class Tag, int D>
hipError_t launch_typed(const AttnParams& p, hipStream_t stream) {
  const dim3 grid(p.nsplit, p.Hkv, p.B);
  if ((p.R + 31) / 32 <= 4)
    hipLaunchKernelGGL((attn_split_kernel<Tag, D, 1, 2>), grid, dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_split_kernel<Tag, D, 2, 1>), grid, dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = p.B * p.K * p.Hq;
  hipLaunchKernelGGL((attn_merge_kernel<Tag, D>), dim3(rows), dim3(kThreads), 0, stream, p);
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
