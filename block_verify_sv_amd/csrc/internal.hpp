// Kernel parameter blocks and launchers of libspecverify (internal; not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "specverify.h"

#include "attention.hpp"
#include "limits.hpp"

namespace sv {

// The whole of sv_verify_attention (validation, planning, launches) on a given workspace;
// `what` names the entry point in launch-failure messages.
sv_status attention_call(const sv_attn_desc* desc, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* page_table, const int32_t* ctx_lens,
                         const uint64_t* block_mask, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream, const char* what);
// Records a status and message for sv_last_error (SV_OK clears it); returns st.
sv_status report(sv_status st, const char* msg);

// ---------------------------------------------------------------- greedy accept
struct GreedyParams {
  const void* logits;
  const int32_t* drafts;      // chain: d_1 .. d_{K-1}; tree: the token of nodes 1 .. K-1
  const int32_t* parents;     // tree: parent of nodes 1 .. K-1
  int32_t* path;              // tree: accepted path [B][K]
  int32_t tree;               // 1: walk a draft tree, 0: a chain
  int32_t* accept_len;
  int32_t* out_tokens;
  int32_t* argmax;
  unsigned long long* keys;   // [B][K][nchunk] packed argmax keys of every chunk
  int32_t B, K, V;
  int32_t chunk;              // vocabulary entries per workgroup
  int32_t nchunk;
};

size_t greedy_workspace_bytes(int B, int K);
int greedy_chunk(int V, sv_dtype dtype);
hipError_t launch_greedy(const GreedyParams& p, sv_dtype dtype, hipStream_t stream);
hipError_t launch_greedy_walk(const GreedyParams& p, hipStream_t stream);   // walk only

// ---------------------------------------------------------------- LM head + greedy
struct LmHeadParams {
  const void* hidden;         // [M][Hd]
  const void* weight;         // [V][Hd], or the packed tile layout when packed != 0
  unsigned long long* part;   // [M][nwg] per-workgroup argmax keys
  int32_t M, V, Hd;
  int32_t nwg;                // argmax workgroups (chosen at launch)
  int32_t packed;
};

size_t lm_head_workspace_bytes(int M, int V);
size_t lm_head_packed_elems(int V, int Hd);   // ceil(V / 32) * 32 * Hd
hipError_t launch_lm_head_pack(const void* weight, void* packed, int V, int Hd,
                               hipStream_t stream);
hipError_t launch_lm_head(const LmHeadParams& p, const GreedyParams& walk, sv_dtype dtype,
                          hipStream_t stream);

// ---------------------------------------------------------------- sampling accept
struct SampleParams {
  const void* target;
  const void* draft;
  const int32_t* drafts;
  int32_t* accept_len;
  int32_t* out_tokens;
  float* part_m;              // [rows][nchunk] chunk maxima of the raw logits
  double* part_s;             // [rows][nchunk] chunk sums of exp((x - m) / T)
  double* race_key;           // [B][race_nchunk][2] chunk winners' keys (residual, p)
  int32_t* race_idx;          // [B][race_nchunk][2]
  int32_t B, K, V;
  int32_t chunk, nchunk;      // vocabulary chunks of the normaliser pass
  int32_t race_chunk, race_nchunk;
  int32_t wait_limit;         // polls a waiting workgroup makes before it gives up
  double inv_t;
  uint64_t seed, offset;
};

// Polls a workgroup waiting on another one's published result makes before it gives up
// (sv_set_wait_limit; 2^18 by default).
int32_t wait_limit();
size_t sample_workspace_bytes(int B, int K, int V);
int sample_chunk(int V);
int sample_race_chunk(int V);
hipError_t launch_sample(const SampleParams& p, sv_dtype dtype, hipStream_t stream);

// ---------------------------------------------------------------- sampling over a tree
// Where the race of a sequence draws from: the stop node u, the children it rejected (m,
// the last one c), u's residual row, Z of the residual before c (1 if m < 2) and the
// log-normalisers of target row u and draft row c.
struct TreeStop {
  double zp, lp, lq;
  int32_t u, c, m, slot;
};

struct TreeSampleParams {
  const void* target;         // [B][K][V]
  const void* draft;          // [B][K-1][V]: row i-1 = the distribution node i was drawn from
  const int32_t* tokens;      // [B][K-1]
  int32_t* accept_len;
  int32_t* out_tokens;        // [B][K]
  int32_t* path;              // [B][K]
  double* zpart;              // [B][K][nz] partial sums of each residual, slot = child node
  double* ztab;               // [B][K] Z of the residual left by rejecting each child
  double* resid;              // [B][nbranch][V] residual of each branching node (fp64)
  float* part_m;              // [B*(2K-1)][4] row parts' maxima (target rows, then draft)
  double* part_s;             // [B*(2K-1)][4] row parts' sums of e^((x - m) / T)
  double* lnorm;              // [B*(2K-1)] row log-normalisers (written by the first pass)
  double* qpair;              // [B][K][64]: [s][c] = q_c(x_s) for c an elder sibling of s
  double* race_key;           // [B][race_nchunk][2]
  int32_t* race_idx;
  TreeStop* stop;             // [B]
  int32_t* fail;              // [B] 1: a wait inside a launch gave up (outputs invalid)
  int32_t B, K, V;
  int32_t nz;                 // residual chunks per row
  int32_t race_chunk, race_nchunk;
  int32_t nbranch;            // nodes with two or more children (at least 1)
  int32_t n_last;             // entries of last_z
  int32_t has_lnorm;          // 1: a residual pass runs and writes lnorm
  int32_t wait_limit;         // polls a waiting workgroup makes before it gives up
  double inv_t;
  uint64_t seed, offset;
  uint64_t elder[kMaxBlock];      // bit i: node i is an elder sibling of node c
  uint64_t younger[kMaxBlock];    // bit i: node i is a younger sibling of node c
  uint64_t zl_mask;               // bit c: c is a second-to-last child (Z folded by the walk)
  int32_t pass_node[kMaxBlock];   // residual-pass words (u | c << 8 | c_prev << 16 | row << 24)
  int8_t parent[kMaxBlock];       // parent of node i (node 0: -1)
  int8_t child_start[kMaxBlock];  // first entry of node u's children in child_list
  int8_t child_count[kMaxBlock];
  int8_t child_list[kMaxBlock];   // children grouped by parent, increasing node order
  int8_t branch_slot[kMaxBlock];  // row of resid of each node with two or more children
  int8_t last_z[kMaxBlock];       // second-to-last child of every branching node
};

// Host side of the plan: where pass j's words start in pass_node and how many it has.
struct TreePassPlan {
  int off[kMaxBlock];
  int n[kMaxBlock];
};

size_t sample_tree_workspace_bytes(int B, int K, int V);
// Points p's scratch arrays into the workspace (p.B, p.K, p.V and the plan's chunk counts
// set).
void carve_sample_tree_workspace(TreeSampleParams& p, void* workspace);
// Fills the plan fields (chunks, tree tables, pass words) of p from the host tree; returns
// the number of residual passes (the largest child count - 1, at least 0).
int plan_sample_tree(TreeSampleParams& p, const int32_t* parents_host, TreePassPlan& plan);
hipError_t launch_sample_tree(const TreeSampleParams& p, const TreePassPlan& plan, int rounds,
                              sv_dtype dtype, hipStream_t stream);

// ---------------------------------------------------------------- latent compressor
struct CompressParams {
  const void* queries;
  const void* feats;
  void* out;
  float* scores;              // [B][C][N] fp32
  uint16_t* weights;          // [B][64][N rounded up to 32] fp16 softmax numerators
  float* rowsum;              // [B][64] sums of the rounded weights
  int32_t B, C, N, D;
  float scale;
};

size_t compress_workspace_bytes(int B, int C, int N);
void compress_bind_workspace(CompressParams& p, void* workspace);
hipError_t launch_compress(const CompressParams& p, hipStream_t stream);

// ---------------------------------------------------------------- KV append
struct AppendParams {
  const void* k_new;
  const void* v_new;
  const int32_t* start;
  const int32_t* page_table;
  void* k_cache;
  void* v_cache;
  int32_t B, n, Hkv, D, P_log2, max_pages, num_pages, elem_bytes;
};

hipError_t launch_kv_append(const AppendParams& p, hipStream_t stream);

// ---------------------------------------------------------------- cycle commit
struct CommitParams {
  const int32_t* accept_len;
  const int32_t* out_tokens;
  int32_t* ctx_lens;
  int32_t* next_anchor;
  int32_t B, K;
};

hipError_t launch_commit(const CommitParams& p, hipStream_t stream);

// ---------------------------------------------------------------- tree commit
struct TreeCompactParams {
  const int32_t* accept_len;
  const int32_t* path;        // [B][K]
  const int32_t* ctx_lens;
  const int32_t* page_table;
  void* k_cache;
  void* v_cache;
  int32_t B, K, Hkv, D, P_log2, max_pages, num_pages, esz;
};

hipError_t launch_tree_compact(const TreeCompactParams& p, hipStream_t stream);

}  // namespace sv
