// Verify-attention parameter block, work plan and launcher (internal; not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "limits.hpp"
#include "specverify.h"

namespace sv {

// ---------------------------------------------------------------- verify attention
struct AttnParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* page_table;
  const int32_t* ctx_lens;
  void* part_o;         // [B][Hkv][nsplit][R][D] partial outputs divided by their own
                        // sum, in the input dtype
  float2* part_ml;      // [B][Hkv][nsplit][R] (running max in log2 units, sum)
  void* out;
  float* lse;
  int32_t B, K, Hq, Hkv, G, R;
  int32_t P_log2, max_pages, num_pages, max_ctx;
  int32_t chunk;        // keys per split
  int32_t nsplit;       // splits allocated per (b, g)
  int32_t nsplit_pad;   // grid spacing of row groups: nsplit, rounded up to a multiple of 8
                        // from 8 splits up or when there are several row groups
  int32_t direct;       // 1: one split per (b, g); the split kernel writes out and lse
  int32_t row_groups;   // row groups per split: ceil(K*G / group rows), a group being
                        // 256 rows for 16-bit data and 128 rows for fp32
  float scale_log2;     // scale * log2(e)
  uint64_t mask[kMaxBlock];
};

struct AttnPlan {
  int chunk;
  int nsplit;
  int row_groups;
  int rows;             // R = K * G
  size_t o_bytes;       // partial outputs (16-byte aligned), then (m, l) pairs
  size_t ws_bytes;
};

AttnPlan plan_attention(const sv_attn_desc& d);
hipError_t launch_attention(const AttnParams& p, int head_dim, sv_dtype dtype,
                            hipStream_t stream);

}  // namespace sv
