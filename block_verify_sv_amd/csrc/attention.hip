// Block-verification attention for gfx950: split-KV pass + online-softmax merge pass.
//
// The target scores all K block rows in one forward over its whole context plus the
// block (VFlash-FM page, "How VFlash-FM works"): for each KV head g the K*G query rows
// of its head group form one dense (K*G) x d tile, so the scores S = Q_g K^T and the
// update O += P V are matrix products and run on MFMA (32x32x16 bf16/f16, 32x32x2 fp32).
//
// Split pass: one workgroup per (sequence b, KV head g, key split s, group of query
// rows), sized so the grid is about one workgroup per compute unit.  Eight waves.  Up to
// 128 rows per KV head, wave (rg, kh) owns query-row block rg (32 rows) and key half kh
// of every 64-key tile, and the two key halves of a row block combine through LDS at the
// end.  With more rows (16-bit data) each wave owns one row block of a 256-row group and
// every key of the tile, so a tile staged in LDS serves twice the rows; fp32 keeps the
// 128-row groups (the full-tile wave would spill).  The split's page ids
// are staged in LDS once, then keys stream in tiles of 64: a ring of four register tiles
// keeps three tiles (96 KB at bf16, d = 128) of global loads in flight while the fourth
// is written to one of two LDS buffers, so the HBM latency is covered without a
// dependent page-table load per tile.  One sequence issues its start-up loads before the
// context length arrives; a batch reads the context length first and lets the splits
// past a shorter sequence's end leave at once.
// With at most 32 query rows per KV head and d = 64 (16-bit), the workgroup is one
// row-block wave pair (128 threads, two-tile ring) so that several share a CU; when every
// (b, g) also fits one split of at most two tiles (the semi-autoregressive block), a pairs
// kernel takes several (b, g) per workgroup and loads the next one's tiles while the
// current one computes.
// Per tile and row block the wave computes S^T = K_tile . Q^T (keys on the MFMA M axis,
// query rows on N, so each lane owns one query row), applies the block mask, runs the
// online softmax in registers, and accumulates O^T = V^T . P^T.
// Output per row: the partial output divided by its own sum, in the input dtype (half the
// bytes of fp32 for 16-bit inputs) and in the accumulator's register order, its
// reference maximum m (log2 units) and sum l.  When every (b, g) has a single split
// those values are the result: the split pass writes the output rows and the lse itself
// and the merge pass is not launched.
//
// Merge pass: one workgroup per (32-wide d block, 32-row block, sequence x KV head); its
// waves read the partial tiles in the same register order (contiguous runs) and combine
// the splits in a fixed order (a split with l = 0, past its sequence's keys or with no
// visible key for the row, is absent; no context length is read):
//   m = max_s m_s, w_s = l_s 2^(m_s - m), out = sum_s w_s O_s / sum_s w_s,
//   lse = (m + log2 sum_s w_s) * ln 2      (O_s: split s's output, already divided by l_s).
#include "attention.hpp"
#include "common.hpp"

namespace sv {
namespace {

constexpr int kTK = 64;           // keys per tile
constexpr float kNegBig = -1.0e30f;
constexpr float kRescale = 8.0f;  // lazy-rescale threshold (log2 units)
#ifndef SV_RING_DEEP
#define SV_RING_DEEP 4
#endif
constexpr int kRingDeep = SV_RING_DEEP;
constexpr int kMaxSplitPages = kMaxSplitKeys / 16 + 2;
// the 128-thread workgroup takes splits of at most this many keys: its page-id stage
// then fits four workgroups' LDS in a CU
constexpr int kMaxSplitKeysSmall = 8192;

// LDS row of key k within a tile: bits 2 and 3 swapped.  With this order the MFMA
// accumulator register r of lane-half h in a 32-key block holds key
// 16*(r/8) + 8*h + (r%8), so the P operand's 8 (16-bit) or 1 (fp32) consecutive
// registers cover consecutive keys and the V^T operand is one contiguous LDS read.
__device__ __forceinline__ int key_row(int k) {
  return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1);
}
__device__ __forceinline__ int key_of_reg(int r, int h) { return 16 * (r >> 3) + 8 * h + (r & 7); }

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// Combine a lane's value with that of lane l ^ 32 through the gfx950 half swap (no LDS
// round trip).  Both halves see the same two operands in the same order.
__device__ __forceinline__ float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

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

// Split kernel.  RG row-group waves x KW key-part waves; wave (rg, kh) owns row blocks
// rg, rg + RG, ... (NRB of them) and keys [32 kh*KBW, 32 (kh+1)*KBW) of every tile.
// LOADS_FIRST: the start-up tile loads go out before the context length is known (one
// sequence: every split is live).  Otherwise (a batch, where the splits past a shorter
// sequence's end are a large part of the grid) the context length is read first and
// those splits leave before loading anything.
template <class Tag, int D, int RG, int NRB, int KW, int RING, bool LOADS_FIRST>
__global__ void __launch_bounds__(64 * RG * KW, 1)
attn_split_kernel(const int32_t* page_table, const void* k_cache, const void* v_cache,
                  const int32_t* ctx_lens,
                  int32_t chunk, int32_t nsplit_pad, int32_t P_log2, int32_t max_pages,
                  int32_t num_pages, int32_t Hkv, const AttnParams p) {
  using S = typename Tag::store_t;
  using Op = typename Mfma<Tag>::op_t;
  constexpr int T = 64 * RG * KW;                // threads
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
  constexpr int K_LDS = 2 * kTK * KROW * SZ;
  constexpr int V_LDS = 2 * D * VROW * SZ;
  constexpr int NSLOT = NRB * (4 * DB + 1);      // 16-byte combine slots per lane
  static_assert(KW == 1 || NSLOT * RG * 64 * 16 <= K_LDS + V_LDS, "combine stage");
  static_assert(K_PER_T >= 1 && V_PER_T >= 1, "tile chunks per thread");

  __shared__ __align__(16) char smem[K_LDS + V_LDS];
  constexpr int MSP = (RG == 1 ? kMaxSplitKeysSmall : kMaxSplitKeys) / 16 + 2;  // page ids
  __shared__ int32_t pg_lds[MSP];
  S* const k_lds = reinterpret_cast<S*>(smem);
  S* const v_lds = reinterpret_cast<S*>(smem + K_LDS);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int rg = wave % RG;                      // row group: row blocks rg + RG*t
  const int kh = wave / RG;                      // key part of each tile
  // blockIdx.x = rgroup * nsplit_pad + s_raw: the row groups of one split are
  // nsplit_pad (then a multiple of 8) workgroups apart, so round-robin dispatch (id i on
  // XCD i mod 8) puts them on one XCD and the later reads of each KV tile come from that
  // XCD's L2.  With a padded grid, split s of (sequence b, KV head g) runs at
  // s_raw = (s + b * Hkv + g) mod nsplit_pad, so that every (b, g) starts on another XCD:
  // otherwise the first splits of all sequences, the ones a short sequence still has,
  // would all land on the first XCDs and overfill them (a batch of 8 sequences put 44
  // live workgroups on the 32 CUs of XCD 0).
  // With LOADS_FIRST no branch comes before the tile loads are issued: an exit taken on
  // a loaded value (the split padding, the context length) would make the compiler wait
  // for that value first and sink every load behind the branch.  A padding workgroup
  // reads pages at its own (clamped) positions, then has no tiles and stores nothing.
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int rgroup = blockIdx.x / nsplit_pad;
  const int s_raw = blockIdx.x - rgroup * nsplit_pad;
  const int rot = (nsplit_pad & 7) == 0 ? (b * Hkv + g) % nsplit_pad : 0;
  const int s = s_raw >= rot ? s_raw - rot : s_raw - rot + nsplit_pad;  // padding ids only
  const bool pad = s >= p.nsplit;                                       // read (clamped) pages
  const int rb0 = rgroup * RG * NRB;               // first row block of this row group

  // ---- start-up.  Nothing below needs the context length until the early-exit test,
  // so every independent load is issued before the first wait and they share one round
  // trip: the page ids of the prologue tiles (read directly from the table, so those
  // tiles' loads follow after a single dependent read), the page ids of the whole split
  // (staged in LDS for the later tiles), the query rows and the block mask.  All of them
  // are unconditional loads at clamped, in-bounds indices: a load under a branch would
  // make the compiler wait for it before the next one.
  const int k0 = s * chunk;
  const int pg0 = k0 >> P_log2;
  const int Pm1 = (1 << P_log2) - 1;
  const int32_t* table = page_table + static_cast<size_t>(b) * max_pages;
  const int last_page = max_pages - 1;
  const int KR = min(Pm1 + 1, kTK);              // keys of one run (see tile staging)
  const int TPR = T * KR / kTK;                  // threads per run
  const int run = tid / TPR;
  const int li = tid - run * TPR;
  const int ntmax = (chunk + kTK - 1) / kTK;     // tiles of a full split
  // the context length is read first, as a scalar load that overlaps the page-table
  // reads; with LOADS_FIRST nothing waits on it until every tile load of the prologue
  // is issued
  const int ctx_raw = ctx_lens[b];
  if constexpr (!LOADS_FIRST) {
    const int ctx0 = ctx_raw < 0 ? 0 : (ctx_raw > p.max_ctx ? p.max_ctx : ctx_raw);
    if (pad || k0 >= ctx0 + p.K) {               // no tiles: an empty (m, l) pair per row
      if (!pad) {
        for (int r = tid; r < p.R; r += T)
          p.part_ml[((static_cast<size_t>(b) * Hkv + g) * p.nsplit + s) * p.R + r] =
              make_float2(kNegBig, 0.0f);
      }
      return;
    }
  }
  int pg_pro[RING - 1];
#pragma unroll
  for (int u = 0; u < RING - 1; ++u) {
    const int pos0 = k0 + min(u, ntmax - 1) * kTK + run * KR;
    pg_pro[u] = table[min(pos0 >> P_log2, last_page)];
  }
  constexpr int NPT = (MSP + T - 1) / T;
  const int npg = min(((k0 + chunk - 1) >> P_log2) - pg0 + 1, max_pages - pg0);
  int pg_all[NPT];
#pragma unroll
  for (int u = 0; u < NPT; ++u) pg_all[u] = table[min(pg0 + tid + u * T, last_page)];
  // query operand (B of S^T = K . Q^T): lane owns query row 32*rb + l32 (padding rows
  // past R read row R-1; their results are never stored)
  Op qop[NRB][KSTEPS];
  uint64_t rmask[NRB];
  bool active[NRB];
#pragma unroll
  for (int t = 0; t < NRB; ++t) {
    const int rb = rb0 + rg + RG * t;
    const int r = min(rb * 32 + l32, p.R - 1);
    active[t] = rb * 32 < p.R;
    const int i = r / p.G;
    const int head = g * p.G + (r - i * p.G);
    const S* qp = static_cast<const S*>(p.q) + ((static_cast<size_t>(b) * p.K + i) * p.Hq + head) * D;
    rmask[t] = p.mask[i];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if constexpr (KPL == 8) {
        qop[t][ks] = *reinterpret_cast<const u32x4*>(qp + ks * 16 + h * 8);
      } else {
        qop[t][ks] = static_cast<float>(qp[h * (D / 2) + ks]);
      }
    }
  }
  const S* kc = static_cast<const S*>(k_cache);
  const S* vc = static_cast<const S*>(v_cache);

  // ---- tile staging: global -> register ring -> LDS.  A 64-key tile is split into
  // runs of KR = min(P, 64) keys that lie in one page; each thread owns a fixed set of
  // 16-byte chunks (K_PER_T of K, V_PER_T of V) inside one run, so a tile costs one
  // page-id lookup per thread and constant offsets from two base pointers.  Loads are
  // branch-free: a run on an unmapped page reads page 0, and a run past the split end
  // reads whatever its (in-pool) page holds; both are zeroed when written to LDS --
  // never at load time, which would make the load wait for its data and empty the ring.
  struct Tile {
    u32x4 k[K_PER_T];
    u32x4 v[V_PER_T];
    int pos0;                                    // first key of this thread's run
    bool page_ok;                                // the run's page id is inside the pool
  };
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
    v_goff[u] = (d << P_log2) + kp * EPC;
    v_loff[u] = d * VROW + run * KR + kp * EPC;
    v_key[u] = run * KR + kp * EPC;              // first key of the chunk in the tile
  }

  // a page holds Hkv heads of P keys x D for K (token-major) and of D x P for V
  // (dim-major): the same element stride per page for both caches
  const uint32_t pstride = static_cast<uint32_t>(Hkv * D) << P_log2;
  const S* const kc_h = kc + (static_cast<size_t>(g * D) << P_log2);
  const S* const vc_h = vc + (static_cast<size_t>(g * D) << P_log2);
  auto load_tile = [&](Tile& r, int kt, int pg) {
    r.pos0 = kt + run * KR;
    r.page_ok = static_cast<unsigned>(pg) < static_cast<unsigned>(num_pages);
    const uint32_t page = r.page_ok ? static_cast<uint32_t>(pg) : 0u;
    const uint32_t slot = static_cast<uint32_t>(r.pos0 & Pm1);
    const size_t poff = static_cast<size_t>(page) * pstride;   // one 32x32 -> 64-bit multiply
    const S* kb = kc_h + poff + slot * D;
    const S* vb = vc_h + poff + slot;
#pragma unroll
    for (int u = 0; u < K_PER_T; ++u) r.k[u] = *reinterpret_cast<const u32x4*>(kb + k_goff[u]);
#pragma unroll
    for (int u = 0; u < V_PER_T; ++u) r.v[u] = *reinterpret_cast<const u32x4*>(vb + v_goff[u]);
  };
  Tile r[RING];
#pragma unroll
  for (int u = 0; u < RING - 1; ++u) load_tile(r[u], k0 + min(u, ntmax - 1) * kTK, pg_pro[u]);
  // every load above is issued before anything waits on the context length: nothing
  // may be moved across this point
  asm volatile("" ::: "memory");

  // ---- the context length: the first value the kernel branches on.  A split past this
  // sequence's keys (or a padding workgroup) keeps k1 = k0: no tiles, no stores.
  const int ctx = ctx_raw < 0 ? 0 : (ctx_raw > p.max_ctx ? p.max_ctx : ctx_raw);
  const int n_keys = ctx + p.K;
  const bool dead = pad || k0 >= n_keys;
  const int k1 = dead ? k0 : min(k0 + chunk, n_keys);
#pragma unroll
  for (int u = 0; u < NPT; ++u) {
    const int i = tid + u * T;
    if (i < npg)
      pg_lds[i] = static_cast<unsigned>(pg_all[u]) < static_cast<unsigned>(num_pages) ? pg_all[u] : -1;
  }
  auto page_of = [&](int kt) {                   // page id of this thread's run of tile kt
    const int pos0 = kt + run * KR;
    return pos0 < k1 ? pg_lds[(pos0 >> P_log2) - pg0] : -1;
  };

  auto store_tile = [&](const Tile& r, int buf, int kt) {
    S* kl = k_lds + buf * kTK * KROW;
    S* vl = v_lds + buf * D * VROW;
    const bool ok = r.page_ok && r.pos0 < k1;
    if (kt + kTK <= k1) {                        // interior tile: zero only unmapped runs
#pragma unroll
      for (int u = 0; u < K_PER_T; ++u)
        *reinterpret_cast<u32x4*>(kl + k_loff[u]) = ok ? r.k[u] : zero4();
#pragma unroll
      for (int u = 0; u < V_PER_T; ++u)
        *reinterpret_cast<u32x4*>(vl + v_loff[u]) = ok ? r.v[u] : zero4();
    } else {                                     // tail tile: also zero keys past k1
      const int left = k1 - kt;
#pragma unroll
      for (int u = 0; u < K_PER_T; ++u)
        *reinterpret_cast<u32x4*>(kl + k_loff[u]) = ok ? r.k[u] : zero4();
#pragma unroll
      for (int u = 0; u < V_PER_T; ++u) {
        u32x4 v = ok ? r.v[u] : zero4();
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
  // O^T += V^T . P^T for row block t over this wave's keys of the tile at vbase
  auto pv = [&](int t, const Op (&pb)[PSW], const S* vbase) {
#pragma unroll
    for (int psi = 0; psi < PSW; ++psi) {
      Op vop[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int ps = kh * PSW + psi;           // MFMA step within the tile
        const S* vrow = vbase + (db * 32 + l32) * VROW;
        if constexpr (KPL == 8) {
          vop[db] = *reinterpret_cast<const u32x4*>(vrow + ps * 16 + h * 8);
        } else {
          vop[db] = static_cast<float>(vrow[32 * (ps >> 4) + key_of_reg(ps & 15, h)]);
        }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[t][db] = Mfma<Tag>::step(vop[db], pb[psi], oacc[t][db]);
    }
  };
  // One step of a wave: S^T for its keys of the tile in LDS buffer buf, mask, online
  // softmax, then P.V.
  auto compute = [&](int buf, int kt) {
    const bool need_mask = (kt + kTK > ctx) || (kt + kTK > k1);
    const S* kbase = k_lds + buf * kTK * KROW;
    f32x16 sacc[NRB][KBW];
    auto scores = [&](int t) {
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
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[t][kbi][e] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) sacc[t][kbi] = Mfma<Tag>::step(kop[ks], qop[t][ks], sacc[t][kbi]);
      }
    };
#pragma unroll
    for (int t = 0; t < NRB; ++t) {
      if (!active[t]) continue;
      scores(t);
      // masked scores are overwritten in place (a separate array would cost a copy of
      // every score on the unmasked path)
      if (need_mask) {
#pragma unroll
        for (int kbi = 0; kbi < KBW; ++kbi) {
          const int kb = kh * KBW + kbi;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            // branch-free: context keys are visible, block key t2 iff bit t2 of the row's
            // mask, nothing at or past the split end
            const int pos = kt + kb * 32 + key_of_reg(r, h);
            const int t2 = pos - ctx;
            const uint32_t bit = static_cast<uint32_t>(rmask[t] >> (t2 & 63)) & 1u;
            const uint32_t vis = static_cast<uint32_t>(pos < k1) & (static_cast<uint32_t>(t2 < 0) | bit);
            sacc[t][kbi][r] = vis ? sacc[t][kbi][r] : -INFINITY;
          }
        }
      }
      float sv[16 * KBW];
#pragma unroll
      for (int kbi = 0; kbi < KBW; ++kbi)
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[kbi * 16 + r] = sacc[t][kbi][r];
      float mt = sv[0];
#pragma unroll
      for (int e = 1; e < 16 * KBW; ++e) mt = fmaxf(mt, sv[e]);
      mt = max_halves(mt);
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
      Op pb[PSW];                                // P^T operands (16-bit: 8 keys a lane)
#pragma unroll
      for (int psi = 0; psi < PSW; ++psi) {
        if constexpr (KPL == 8) {
          const float* pv8 = &sv[psi * 8];
          pb[psi] = u32x4{Tag::pack2(pv8[0], pv8[1]), Tag::pack2(pv8[2], pv8[3]),
                          Tag::pack2(pv8[4], pv8[5]), Tag::pack2(pv8[6], pv8[7])};
        } else {
          pb[psi] = sv[psi];
        }
      }
      pv(t, pb, v_lds + buf * D * VROW);
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
  // The page id of each ring load is read from LDS one step ahead, so its LDS round
  // trip overlaps a step's math instead of delaying the load issue.
  int pg_next = page_of(tile_at(RING - 1));
  auto step = [&](int j, Tile& rl, const Tile& rs, int buf) {
    load_tile(rl, tile_at(j + RING - 1), pg_next);
    pg_next = page_of(tile_at(j + RING));
    compute(buf, k0 + j * kTK);
    if (j + 1 < nt) store_tile(rs, buf ^ 1, k0 + (j + 1) * kTK);
    __syncthreads();
  };
  store_tile(r[0], 0, k0);
  __syncthreads();
  if (dead) {                                    // workgroup-uniform, after the last barrier use
    // a real split past this sequence's keys leaves an empty (m, l) pair for each row,
    // which is all the merge reads of it (its O rows keep whatever the workspace held)
    if (!pad) {
      for (int r = tid; r < p.R; r += T)
        p.part_ml[((static_cast<size_t>(b) * Hkv + g) * p.nsplit + s) * p.R + r] =
            make_float2(kNegBig, 0.0f);
    }
    return;
  }
  for (int j0 = 0; j0 < nt; j0 += RING) {
#pragma unroll
    for (int u = 0; u < RING; ++u) {
      const int j = j0 + u;
      if (j >= nt) break;
      step(j, r[(u + RING - 1) % RING], r[(u + 1) % RING], j & 1);
    }
  }

  // ---- the row's sum over both lane halves, then (KW == 2) the two key-part waves of
  // a row group combine through LDS (the tile buffers are free after the last barrier).
  // The pair splits the d blocks: each wave stages the half its partner finishes, then
  // combines and stores its own half, so both waves share the epilogue's work.  Both
  // compute the combined (m, l) from the same two pairs (m = max of the two, each side
  // weighted by exp2 of its distance to m); the kh = 0 wave stores it.
#pragma unroll
  for (int t = 0; t < NRB; ++t) l_run[t] = sum_halves(l_run[t]);
  // Wave kh finishes d blocks kh*HB .. kh*HB+HB-1; its results end up in oacc[t][0..HB)
  // (registers are picked by value, never by a runtime index).
  constexpr int HB = KW == 2 ? DB / 2 : DB;
  if constexpr (KW == 2) {
    // staged as [slot][row group][lane] 16-byte slots: every LDS access of a wave is one
    // contiguous, conflict-free 1 KB run; wave kh writes slots kh*4*HB + 4*j + q4 (quad q4
    // of the j-th d block of the half its partner finishes), and slot 4*DB holds the
    // (m, l) of key part kh in its 8-byte half kh
    f32x4* stage = reinterpret_cast<f32x4*>(smem);
    float2* stage_ml = reinterpret_cast<float2*>(smem);
    auto slot = [&](int t, int c) { return ((t * (4 * DB + 1) + c) * RG + rg) * 64 + lane; };
    const bool lo_half = kh == 0;
#pragma unroll
    for (int t = 0; t < NRB; ++t) {
      if (!active[t]) continue;
#pragma unroll
      for (int j = 0; j < HB; ++j)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 lo = {oacc[t][j][4 * q4], oacc[t][j][4 * q4 + 1], oacc[t][j][4 * q4 + 2],
                            oacc[t][j][4 * q4 + 3]};
          const f32x4 hi = {oacc[t][j + HB][4 * q4], oacc[t][j + HB][4 * q4 + 1],
                            oacc[t][j + HB][4 * q4 + 2], oacc[t][j + HB][4 * q4 + 3]};
          stage[slot(t, kh * 4 * HB + 4 * j + q4)] = lo_half ? hi : lo;
        }
      stage_ml[2 * slot(t, 4 * DB) + kh] = make_float2(m_run[t], l_run[t]);
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NRB; ++t) {
      if (!active[t]) continue;
      const float2 ml2 = stage_ml[2 * slot(t, 4 * DB) + 1 - kh];
      const float m = fmaxf(m_run[t], ml2.x);
      const float a1 = fast_exp2((m_run[t] - m) * c2), a2 = fast_exp2((ml2.x - m) * c2);
      m_run[t] = m;
      l_run[t] = l_run[t] * a1 + ml2.y * a2;
#pragma unroll
      for (int j = 0; j < HB; ++j)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 o2 = stage[slot(t, (1 - kh) * 4 * HB + 4 * j + q4)];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float own = lo_half ? oacc[t][j][4 * q4 + e] : oacc[t][j + HB][4 * q4 + e];
            oacc[t][j][4 * q4 + e] = own * a1 + o2[e] * a2;
          }
        }
    }
  }

  // ---- partial results: O / l in the input dtype, (m, l) in fp32.  O is kept in the
  // accumulator's own order, [b, g][row block][d block][register quad][split][lane] x 4
  // consecutive d values: each store instruction of a wave writes one contiguous run
  // (512 bytes for 16-bit data), and the merge reads every split of one (row block,
  // d block, quad) as a single contiguous stretch.
  // With a single split per (b, g) (p.direct) the same values are the result: they go
  // straight to the output rows [b][i][head][d] and the lse, and no merge runs.
  const int RBT = (p.R + 31) >> 5;
  const size_t bg = static_cast<size_t>(b) * Hkv + g;
#pragma unroll
  for (int t = 0; t < NRB; ++t) {
    if (!active[t]) continue;
    const int rb = rb0 + rg + RG * t;
    const int r = rb * 32 + l32;
    if (r < p.R && p.direct) {
      const float inv = l_run[t] > 0.0f ? 1.0f / l_run[t] : 0.0f;
      const int i = r / p.G;
      const size_t orow = (static_cast<size_t>(b) * p.K + i) * p.Hq + g * p.G + (r - i * p.G);
#pragma unroll
      for (int j = 0; j < HB; ++j) {
        const int db = (KW == 2 ? kh * HB : 0) + j;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float o[4] = {oacc[t][j][4 * q4], oacc[t][j][4 * q4 + 1],
                              oacc[t][j][4 * q4 + 2], oacc[t][j][4 * q4 + 3]};
          S* dst = static_cast<S*>(p.out) + orow * D + db * 32 + 8 * q4 + 4 * h;
          if constexpr (SZ == 2) {
            const uint2 v = {Tag::pack2(o[0] * inv, o[1] * inv), Tag::pack2(o[2] * inv, o[3] * inv)};
            *reinterpret_cast<uint2*>(dst) = v;
          } else {
            *reinterpret_cast<f32x4*>(dst) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
          }
        }
      }
      if (p.lse && h == 0 && kh == 0)
        p.lse[orow] = (m_run[t] * c2 + log2f(l_run[t])) * 0.69314718055994531f;
    } else if (r < p.R) {
      const float inv = l_run[t] > 0.0f ? 1.0f / l_run[t] : 0.0f;
#pragma unroll
      for (int j = 0; j < HB; ++j) {
        const int db = (KW == 2 ? kh * HB : 0) + j;     // runtime only in the address
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float o[4] = {oacc[t][j][4 * q4], oacc[t][j][4 * q4 + 1],
                              oacc[t][j][4 * q4 + 2], oacc[t][j][4 * q4 + 3]};
          S* dst = static_cast<S*>(p.part_o) +
                   ((((bg * RBT + rb) * DB + db) * 4 + q4) * p.nsplit + s) * 256 + lane * 4;
          if constexpr (SZ == 2) {
            const uint2 v = {Tag::pack2(o[0] * inv, o[1] * inv), Tag::pack2(o[2] * inv, o[3] * inv)};
            *reinterpret_cast<uint2*>(dst) = v;
          } else {
            *reinterpret_cast<f32x4*>(dst) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
          }
        }
      }
      if (h == 0 && kh == 0) {
        const size_t rowid = (bg * p.nsplit + s) * p.R + r;
        p.part_ml[rowid] = make_float2(m_run[t] * c2, l_run[t]);   // m in log2 units
      }
    }
  }
}

// Pairs kernel: several (sequence, KV head) pairs per workgroup, each pair's keys (at most
// two 64-key tiles, such as the semi-autoregressive block's compressed rows plus its
// slots) in one split whose output is written directly.  While a pair computes, the next
// pair's two tiles are already loading into registers (and the pair after it has its
// page ids and query rows loading), so the start-up round trips of every pair but the
// first hide under work.  One row block of at most 32 rows, two key-half waves, 16-bit
// data; the per-tile math is the split kernel's.
template <class Tag, int D>
__global__ void __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_pairs_kernel(const int32_t* page_table, const void* k_cache, const void* v_cache,
                  const int32_t* ctx_lens, int32_t npairs, int32_t P_log2, int32_t max_pages,
                  int32_t num_pages, int32_t Hkv, const AttnParams p) {
  using S = typename Tag::store_t;
  using Op = typename Mfma<Tag>::op_t;
  static_assert(Tag::kBytes == 2 && Tag::KPL == 8, "16-bit data");
  constexpr int T = 128;
  constexpr int EPC = 8;
  constexpr int KROW = D + EPC;
  constexpr int VROW = kTK + EPC;
  constexpr int CPK = D / EPC;
  constexpr int K_PER_T = kTK * D / EPC / T;
  constexpr int V_PER_T = D * kTK / EPC / T;
  constexpr int KSTEPS = D / 16;
  constexpr int PSW = 2;                         // MFMA steps over a wave's 32 keys
  constexpr int DB = D / 32;
  constexpr int HB = DB / 2;
  constexpr int NT = 2;                          // tiles per pair
  constexpr int K_LDS = NT * kTK * KROW * 2;
  constexpr int V_LDS = NT * D * VROW * 2;
  static_assert((4 * DB + 1) * 64 * 16 <= K_LDS + V_LDS, "combine stage");
  __shared__ __align__(16) char smem[K_LDS + V_LDS];
  S* const k_lds = reinterpret_cast<S*>(smem);
  S* const v_lds = reinterpret_cast<S*>(smem + K_LDS);

  const int tid = threadIdx.x;
  const int kh = __builtin_amdgcn_readfirstlane(tid >> 6);   // key half of every tile
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int Pm1 = (1 << P_log2) - 1;
  const int last_page = max_pages - 1;
  const int KR = min(Pm1 + 1, kTK);
  const int TPR = T * KR / kTK;
  const int run = tid / TPR;
  const int li = tid - run * TPR;
  const int KGR = KR / EPC;
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
    v_goff[u] = (d << P_log2) + kp * EPC;
    v_loff[u] = d * VROW + run * KR + kp * EPC;
    v_key[u] = run * KR + kp * EPC;
  }
  const uint32_t pstride = static_cast<uint32_t>(Hkv * D) << P_log2;
  const S* const kc = static_cast<const S*>(k_cache);
  const S* const vc = static_cast<const S*>(v_cache);
  const float c2 = p.scale_log2;
  const float resc = kRescale / c2;
  const int r = min(l32, p.R - 1);               // this lane's query row
  const int ri = r / p.G;
  const uint64_t rmask = p.mask[ri];

  // per pair: where it is and what its loads need (all loads unconditional, clamped)
  struct Meta {
    int b, g, ctx;
    int pg[NT];
  };
  auto meta = [&](int q, Meta& m) {
    const int qq = min(q, npairs - 1);
    m.b = qq / Hkv;
    m.g = qq - m.b * Hkv;
    m.ctx = ctx_lens[m.b];
    const int32_t* table = page_table + static_cast<size_t>(m.b) * max_pages;
#pragma unroll
    for (int t = 0; t < NT; ++t) m.pg[t] = table[min((t * kTK + run * KR) >> P_log2, last_page)];
  };
  auto load_q = [&](const Meta& m, Op (&qo)[KSTEPS]) {
    const int head = m.g * p.G + (r - ri * p.G);
    const S* qp = static_cast<const S*>(p.q) + ((static_cast<size_t>(m.b) * p.K + ri) * p.Hq + head) * D;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qo[ks] = *reinterpret_cast<const u32x4*>(qp + ks * 16 + h * 8);
  };
  u32x4 tk[NT][K_PER_T], tv[NT][V_PER_T];
  bool pok[NT];
  auto load_tiles = [&](const Meta& m) {
    const S* kc_h = kc + (static_cast<size_t>(m.g * D) << P_log2);
    const S* vc_h = vc + (static_cast<size_t>(m.g * D) << P_log2);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      pok[t] = static_cast<unsigned>(m.pg[t]) < static_cast<unsigned>(num_pages);
      const uint32_t page = pok[t] ? static_cast<uint32_t>(m.pg[t]) : 0u;
      const uint32_t slot = static_cast<uint32_t>((t * kTK + run * KR) & Pm1);
      const size_t poff = static_cast<size_t>(page) * pstride;
      const S* kb = kc_h + poff + slot * D;
      const S* vb = vc_h + poff + slot;
#pragma unroll
      for (int u = 0; u < K_PER_T; ++u) tk[t][u] = *reinterpret_cast<const u32x4*>(kb + k_goff[u]);
#pragma unroll
      for (int u = 0; u < V_PER_T; ++u) tv[t][u] = *reinterpret_cast<const u32x4*>(vb + v_goff[u]);
    }
  };

  Meta cur, nxt;
  Op qcur[KSTEPS], qnxt[KSTEPS];
  const int stride = gridDim.x;
  int q = blockIdx.x;
  meta(q, cur);
  load_tiles(cur);
  load_q(cur, qnxt);
  meta(q + stride, nxt);
  for (; q < npairs; q += stride) {
    const int ctx = cur.ctx < 0 ? 0 : (cur.ctx > p.max_ctx ? p.max_ctx : cur.ctx);
    const int nk = ctx + p.K;                    // at most NT tiles (checked at launch)
    // ---- both tiles into LDS (keys past nk zeroed in V; their scores are masked)
    __syncthreads();                             // the previous pair's epilogue is done with LDS
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      S* kl = k_lds + t * kTK * KROW;
      S* vl = v_lds + t * D * VROW;
      const bool ok = pok[t] && t * kTK + run * KR < nk;
      const int left = nk - t * kTK;
#pragma unroll
      for (int u = 0; u < K_PER_T; ++u)
        *reinterpret_cast<u32x4*>(kl + k_loff[u]) = ok ? tk[t][u] : zero4();
#pragma unroll
      for (int u = 0; u < V_PER_T; ++u) {
        u32x4 v = ok ? tv[t][u] : zero4();
        v = keep16(v, left - v_key[u]);
        *reinterpret_cast<u32x4*>(vl + v_loff[u]) = v;
      }
    }
    __syncthreads();
    // ---- the next pair's tiles load while this one computes; the one after that
    // fetches its page ids and query rows
    const int ub = cur.b, ug = cur.g;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qcur[ks] = qnxt[ks];
    load_tiles(nxt);
    load_q(nxt, qnxt);
    cur = nxt;
    meta(q + 2 * stride, nxt);

    float m_run = kNegBig, l_run = 0.0f;
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][e] = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int kt = t * kTK;
      if (kt >= nk) break;                       // workgroup-uniform
      const S* krow = k_lds + t * kTK * KROW + (kh * 32 + l32) * KROW;
      Op kop[KSTEPS];
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) kop[ks] = *reinterpret_cast<const u32x4*>(krow + ks * 16 + h * 8);
      f32x16 sacc;
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[e] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) sacc = Mfma<Tag>::step(kop[ks], qcur[ks], sacc);
      // visible: context keys, block key t2 iff bit t2 of the row's mask, nothing past nk
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int pos = kt + kh * 32 + key_of_reg(rr, h);
        const int t2 = pos - ctx;
        const uint32_t bit = static_cast<uint32_t>(rmask >> (t2 & 63)) & 1u;
        const uint32_t vis = static_cast<uint32_t>(pos < nk) & (static_cast<uint32_t>(t2 < 0) | bit);
        sacc[rr] = vis ? sacc[rr] : -INFINITY;
      }
      float mt = sacc[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mt = fmaxf(mt, sacc[e]);
      mt = max_halves(mt);
      if (__any(mt > m_run + resc)) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = fast_exp2((m_run - m_new) * c2);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
      }
      const float mneg = -m_run * c2;
      float sv[16];
      float psum = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sv[e] = fast_exp2(fmaf(sacc[e], c2, mneg));
        psum += sv[e];
      }
      l_run += psum;
#pragma unroll
      for (int psi = 0; psi < PSW; ++psi) {
        const float* pv8 = &sv[psi * 8];
        const Op pb = u32x4{Tag::pack2(pv8[0], pv8[1]), Tag::pack2(pv8[2], pv8[3]),
                            Tag::pack2(pv8[4], pv8[5]), Tag::pack2(pv8[6], pv8[7])};
        const int ps = kh * PSW + psi;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const S* vrow = v_lds + t * D * VROW + (db * 32 + l32) * VROW;
          const Op vop = *reinterpret_cast<const u32x4*>(vrow + ps * 16 + h * 8);
          oacc[db] = Mfma<Tag>::step(vop, pb, oacc[db]);
        }
      }
    }
    // ---- the key halves combine through LDS (as in the split kernel), then the rows go
    // straight to the output
    l_run = sum_halves(l_run);
    __syncthreads();                             // both waves are done reading the tiles
    f32x4* stage = reinterpret_cast<f32x4*>(smem);
    float2* stage_ml = reinterpret_cast<float2*>(smem);
    auto slot = [&](int c) { return c * 64 + lane; };
    const bool lo_half = kh == 0;
#pragma unroll
    for (int j = 0; j < HB; ++j)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 lo = {oacc[j][4 * q4], oacc[j][4 * q4 + 1], oacc[j][4 * q4 + 2], oacc[j][4 * q4 + 3]};
        const f32x4 hi = {oacc[j + HB][4 * q4], oacc[j + HB][4 * q4 + 1], oacc[j + HB][4 * q4 + 2],
                          oacc[j + HB][4 * q4 + 3]};
        stage[slot(kh * 4 * HB + 4 * j + q4)] = lo_half ? hi : lo;
      }
    stage_ml[2 * slot(4 * DB) + kh] = make_float2(m_run, l_run);
    __syncthreads();
    const float2 ml2 = stage_ml[2 * slot(4 * DB) + 1 - kh];
    const float mm = fmaxf(m_run, ml2.x);
    const float a1 = fast_exp2((m_run - mm) * c2), a2 = fast_exp2((ml2.x - mm) * c2);
    const float L = l_run * a1 + ml2.y * a2;
#pragma unroll
    for (int j = 0; j < HB; ++j)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 o2 = stage[slot((1 - kh) * 4 * HB + 4 * j + q4)];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float own = lo_half ? oacc[j][4 * q4 + e] : oacc[j + HB][4 * q4 + e];
          oacc[j][4 * q4 + e] = own * a1 + o2[e] * a2;
        }
      }
    if (l32 < p.R) {
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      const size_t orow = (static_cast<size_t>(ub) * p.K + ri) * p.Hq + ug * p.G + (r - ri * p.G);
#pragma unroll
      for (int j = 0; j < HB; ++j) {
        const int db = kh * HB + j;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          S* dst = static_cast<S*>(p.out) + orow * D + db * 32 + 8 * q4 + 4 * h;
          const uint2 v = {Tag::pack2(oacc[j][4 * q4] * inv, oacc[j][4 * q4 + 1] * inv),
                           Tag::pack2(oacc[j][4 * q4 + 2] * inv, oacc[j][4 * q4 + 3] * inv)};
          *reinterpret_cast<uint2*>(dst) = v;
        }
      }
      if (p.lse && h == 0 && kh == 0) p.lse[orow] = (mm * c2 + log2f(L)) * 0.69314718055994531f;
    }
  }
}

// Four consecutive partial-output elements as floats.
template <class Tag>
__device__ __forceinline__ f32x4 load4(const typename Tag::store_t* src) {
  if constexpr (Tag::kBytes == 2) {
    const uint2 w = *reinterpret_cast<const uint2*>(src);
    return f32x4{Tag::to_f32(static_cast<uint16_t>(w.x)), Tag::to_f32(static_cast<uint16_t>(w.x >> 16)),
                 Tag::to_f32(static_cast<uint16_t>(w.y)), Tag::to_f32(static_cast<uint16_t>(w.y >> 16))};
  } else {
    return *reinterpret_cast<const f32x4*>(src);
  }
}

// Merge: one workgroup per (d block of 32 x register quad, row block of 32, sequence b x
// KV head g).  Lane l owns row 32*rb + l%32 and the 4 d values 8q + 4(l/32) .. +3 of the
// d block -- the partial layout's own order, so a wave's load of one split is one
// contiguous 512-byte run.  Wave w folds splits w, w+8, ... in batches of BATCH (all
// loads of a batch in flight; 8 when a pair has more than 32 splits, else 4, so few
// loads go to clamped repeats) with a running maximum; the eight wave states are
// combined in wave order through LDS.  Registers are given to the loads in flight
// rather than to occupancy.
constexpr int kMergeWaves = 8;

template <class Tag, int D, int BATCH>
__global__ void __launch_bounds__(kMergeWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 2)))
attn_merge_kernel(const void* part_o, const float2* part_ml, int32_t R, int32_t B, int32_t Hkv,
                  int32_t nsplit, const AttnParams p) {
  using S = typename Tag::store_t;
  constexpr int DB = D / 32;
  __shared__ f32x4 st[2][kMergeWaves][64];       // accumulator quad, (m, l) per lane

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int lane = tid & 63;
  const int h = lane >> 5;
  // Workgroups go to the 8 XCDs round-robin by linear id.  The NX workgroups of one
  // (row block, b * Hkv + g) pair -- one per (d block, register quad) -- get ids of one
  // residue mod 8, so that pair's (m, l) rows are fetched into one XCD's L2 instead of
  // into all eight.  Ids past the last pair (the pair count rounded up to 8) exit.
  // The merge reads no context length: every real split leaves an (m, l) pair for each
  // row, an empty one (l = 0) when it lies past its sequence's keys, so no load waits on
  // another and no branch comes before the loads (ids past the last pair read the last
  // pair and leave after the loads).
  constexpr int NX = 4 * DB;
  const int RBT = (R + 31) >> 5;
  const int slot = blockIdx.x >> 3;
  const int npairs = RBT * B * Hkv;
  const int pair_raw = (slot / NX) * 8 + (blockIdx.x & 7);
  const bool live = pair_raw < npairs;
  const int pair = live ? pair_raw : npairs - 1;
  const int x = slot - (slot / NX) * NX;
  const int db = x >> 2;
  const int q = x & 3;
  const int rb = pair % RBT;
  const int bg = pair / RBT;                     // b * Hkv + g
  const int b = bg / Hkv;
  const int g = bg - b * Hkv;
  const int r = rb * 32 + (lane & 31);
  const bool valid = r < R;                      // padding rows of the last row block
  const S* const po = static_cast<const S*>(part_o) +
                      ((((static_cast<size_t>(bg) * RBT + rb) * DB + db) * 4 + q) * nsplit) * 256 + lane * 4;
  const float2* const pml = part_ml + static_cast<size_t>(bg) * nsplit * R + min(r, R - 1);

  float m_w = kNegBig, l_w = 0.0f;
  f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // Loads cover every allocated split.  They are unconditional, at clamped in-bounds
  // indices -- a load under a branch would be waited for before the next one.  A split
  // with l = 0 (past its sequence's end; its O rows are stale workspace and may hold
  // anything) adds nothing: its O is replaced by zeros before it is weighted.
  for (int s0 = wave; s0 < nsplit; s0 += kMergeWaves * BATCH) {
    float2 ml[BATCH];
    f32x4 o[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const size_t sp = static_cast<size_t>(min(s0 + u * kMergeWaves, nsplit - 1));
      ml[u] = pml[sp * R];
      o[u] = load4<Tag>(po + sp * 256);
    }
    asm volatile("" ::: "memory");               // the whole batch is in flight before any use
#pragma unroll
    for (int u = 0; u < BATCH; ++u)
      if (s0 + u * kMergeWaves >= nsplit || !(ml[u].y > 0.0f)) {
        ml[u] = make_float2(kNegBig, 0.0f);
        o[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    float bm = m_w;
#pragma unroll
    for (int u = 0; u < BATCH; ++u) bm = fmaxf(bm, ml[u].x);
    const float a = fast_exp2(m_w - bm);
    m_w = bm;
    l_w *= a;
    acc *= a;
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const float w = ml[u].y * fast_exp2(ml[u].x - bm);   // 0 for absent / empty splits
      l_w += w;
      acc += w * o[u];
    }
  }
  st[0][wave][lane] = acc;
  st[1][wave][lane] = f32x4{m_w, l_w, 0.0f, 0.0f};
  __syncthreads();
  if (!live || wave != 0 || !valid) return;

  float M = kNegBig;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) M = fmaxf(M, st[1][w][lane][0]);
  float L = 0.0f;
  f32x4 o = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) {
    const f32x4 ml = st[1][w][lane];
    const float a = ml[1] > 0.0f ? fast_exp2(ml[0] - M) : 0.0f;
    L += ml[1] * a;
    o += a * st[0][w][lane];
  }
  const float inv = 1.0f / L;
  const int i = r / p.G;
  const int hq = g * p.G + (r - i * p.G);
  S* out = static_cast<S*>(p.out) + ((static_cast<size_t>(b) * p.K + i) * p.Hq + hq) * D +
           db * 32 + 8 * q + 4 * h;
  if constexpr (Tag::kBytes == 2) {
    *reinterpret_cast<uint2*>(out) = uint2{Tag::pack2(o[0] * inv, o[1] * inv), Tag::pack2(o[2] * inv, o[3] * inv)};
  } else {
    *reinterpret_cast<f32x4*>(out) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
  }
  if (p.lse && x == 0 && h == 0)                 // the (d block 0, quad 0) workgroup
    p.lse[(static_cast<size_t>(b) * p.K + i) * p.Hq + hq] = (M + log2f(L)) * 0.69314718055994531f;
}

template <class Tag, int D>
hipError_t launch_typed(const AttnParams& p, hipStream_t stream) {
  // 4 row-group waves x 2 key halves, one row block each (512 threads, two waves per
  // SIMD), a deep register ring for 16-bit data.  More than 4 row blocks (K*G > 128)
  // run as row groups of the same split: 8 row-block waves over whole tiles (256 rows)
  // for 16-bit data, up to four groups of 128 rows for fp32.  One sequence issues its
  // start-up loads before reading its context length; a batch reads it first.
  const dim3 grid(p.nsplit_pad * p.row_groups, p.Hkv, p.B);
#define SPLIT_ARGS p.page_table, p.k_cache, p.v_cache, p.ctx_lens, p.chunk, p.nsplit_pad, \
                   p.P_log2, p.max_pages, p.num_pages, p.Hkv, p
#define MERGE_ARGS p.part_o, p.part_ml, p.R, p.B, p.Hkv, p.nsplit, p
  constexpr int RING = Tag::kBytes == 2 ? kRingDeep : 2;
  bool launched = false;
  if constexpr (D == 64 && Tag::kBytes == 2) {
    // at most one row block and two tiles per (b, g) (the semi-autoregressive block):
    // workgroups of one row-block wave pair that take several pairs each
    if (p.direct && p.R <= 32 && p.max_ctx + p.K <= 2 * kTK) {
      const int npairs = p.B * p.Hkv;
      const int nwg = npairs < 4 * kNumCUs ? npairs : 4 * kNumCUs;
      hipLaunchKernelGGL((attn_pairs_kernel<Tag, D>), dim3(nwg), dim3(128), 0, stream,
                         p.page_table, p.k_cache, p.v_cache, p.ctx_lens, npairs, p.P_log2,
                         p.max_pages, p.num_pages, p.Hkv, p);
      return hipGetLastError();
    }
    // at most one row block per KV head (the semi-autoregressive block: 5 rows, G = 1):
    // one row-block wave pair of 128 threads, four workgroups per CU
    launched = p.R <= 32 && p.chunk <= kMaxSplitKeysSmall;
    if (launched)
      hipLaunchKernelGGL((attn_split_kernel<Tag, D, 1, 1, 2, 2, false>), grid, dim3(128), 0, stream, SPLIT_ARGS);
  }
  if constexpr (Tag::kBytes == 2) {
    if (!launched && p.R > 128) {
      if (p.B == 1)
        hipLaunchKernelGGL((attn_split_kernel<Tag, D, 8, 1, 1, RING, true>), grid, dim3(512), 0, stream, SPLIT_ARGS);
      else
        hipLaunchKernelGGL((attn_split_kernel<Tag, D, 8, 1, 1, RING, false>), grid, dim3(512), 0, stream, SPLIT_ARGS);
      launched = true;
    }
  }
  if (!launched) {
    if (p.B == 1)
      hipLaunchKernelGGL((attn_split_kernel<Tag, D, 4, 1, 2, RING, true>), grid, dim3(512), 0, stream, SPLIT_ARGS);
    else
      hipLaunchKernelGGL((attn_split_kernel<Tag, D, 4, 1, 2, RING, false>), grid, dim3(512), 0, stream, SPLIT_ARGS);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.direct) return e;
  const int pairs = (p.R + 31) / 32 * p.B * p.Hkv;
  const dim3 mgrid(D / 32 * 4 * ((pairs + 7) / 8 * 8));
  if (p.nsplit > 32)
    hipLaunchKernelGGL((attn_merge_kernel<Tag, D, 8>), mgrid, dim3(kMergeWaves * 64), 0, stream, MERGE_ARGS);
  else
    hipLaunchKernelGGL((attn_merge_kernel<Tag, D, 4>), mgrid, dim3(kMergeWaves * 64), 0, stream, MERGE_ARGS);
#undef SPLIT_ARGS
#undef MERGE_ARGS
  return hipGetLastError();
}

}  // namespace

AttnPlan plan_attention(const sv_attn_desc& d) {
  AttnPlan pl;
  const int64_t n_max = static_cast<int64_t>(d.max_ctx) + d.block;
  pl.rows = d.block * (d.num_q_heads / d.num_kv_heads);
  // a workgroup holds 4 row blocks of 32 (two key halves each), or 8 (whole tiles) when
  // a 16-bit head group has more than 128 rows
  const int group_rows = (d.dtype != SV_F32 && pl.rows > 128) ? 256 : 128;
  pl.row_groups = (pl.rows + group_rows - 1) / group_rows;
  int64_t chunk = d.split_keys;
  if (chunk == 0) {
    // at most one workgroup per compute unit: total (context + block) keys over all KV
    // heads and row groups, spread in whole 64-key tiles, and no longer than the longest
    // sequence rounded up to min(P, 64) keys.  Every sequence's last split may be
    // partial, so the keys are spread over the CUs left after one such split per
    // (sequence, KV head, row group).  One sequence fills those CUs; a batch, whose
    // per-sequence lengths are not known here, is spread over three quarters of them
    // (sweeps of 8-sequence batches over the split size ran fastest with 150-200 live
    // workgroups: 80.8 -> 60.7, 82.0 -> 76.4 and 80.8 -> 65 us per pass for three
    // context mixes, against the 272-296 live workgroups of a full spread).
    const int64_t gran = d.page_size < 64 ? d.page_size : 64;
    const int64_t ctx_sum =
        d.sum_ctx_hint > 0 ? d.sum_ctx_hint : static_cast<int64_t>(d.batch) * d.max_ctx;
    const int64_t work =
        (ctx_sum + static_cast<int64_t>(d.batch) * d.block) * d.num_kv_heads * pl.row_groups;
    const int64_t tails = static_cast<int64_t>(d.batch) * d.num_kv_heads * pl.row_groups;
    const int64_t target = d.batch > 1 ? kNumCUs * 3 / 4 : kNumCUs;
    const int64_t cus = tails <= target / 2 ? target - tails : target;
    chunk = (work + cus - 1) / cus;
    // whole 64-key tiles: a split's last tile costs a full step however few keys it
    // holds, so rounding up to the tile keeps the step count and needs fewer splits
    chunk = (chunk + 63) / 64 * 64;
    if (chunk < 64) chunk = 64;
    const int64_t cap = (n_max + gran - 1) / gran * gran;
    if (chunk > cap) chunk = cap;
    if (chunk > kMaxSplitKeys) chunk = kMaxSplitKeys;
  }
  pl.chunk = static_cast<int>(chunk);
  pl.nsplit = static_cast<int>((n_max + chunk - 1) / chunk);
  const size_t esz = d.dtype == SV_F32 ? 4 : 2;
  const size_t units = static_cast<size_t>(d.batch) * d.num_kv_heads * pl.nsplit;
  // partial outputs are stored in whole 32-row blocks (the accumulator tile order)
  const size_t padded_rows = static_cast<size_t>((pl.rows + 31) / 32 * 32);
  pl.o_bytes = (units * padded_rows * d.head_dim * esz + 15) / 16 * 16;
  pl.ws_bytes = pl.o_bytes + units * pl.rows * sizeof(float2);
  return pl;
}

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
