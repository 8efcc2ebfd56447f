/*
 * libspecverify -- one-pass block verification for lossless speculative decoding.
 *
 * A drafter proposes a block of K tokens (the anchor, i.e. the last committed
 * token, followed by K-1 drafts); the unchanged target scores every block
 * position in one forward over its whole context plus the block, and an
 * acceptance rule decides how many drafts to keep (VFlash-FM page, "How VFlash-FM
 * works", cycle figure and caption).  This library runs the data-parallel part
 * of that step on one AMD Instinct MI355X (gfx950):
 *
 *   sv_verify_attention  block-causal grouped-query attention of the K block rows
 *                        over a paged KV cache (split-KV pass + merge pass)
 *   sv_accept_greedy     longest prefix matching the target's argmax + correction
 *   sv_accept_sample     min(1, p/q) acceptance with a residual resample, driven
 *                        by counter-based Philox4x64-10 uniforms
 *   sv_latent_compress   softmax(C . F^T) . F latent visual compressor
 *   sv_kv_append         write new K/V rows into the paged cache
 *   sv_commit            close a cycle: grow the context, pick the next anchor
 *   sv_accept_greedy_tree  greedy verification of a draft tree (walk from the anchor)
 *   sv_accept_sample_tree  sampling verification of a draft tree (recursive rejection)
 *   sv_commit_tree       close a tree cycle: move the accepted path's K/V into place
 *   sv_lm_head_greedy    the target's LM head fused with greedy acceptance
 *   sv_lm_head_pack, sv_lm_head_greedy_packed  the same over a weight packed once
 *
 * Conventions for every call
 *   - Array arguments are DEVICE pointers unless stated otherwise.  The caller
 *     owns all memory, including the workspace; the library never allocates,
 *     frees or synchronises.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  Outputs are valid once the stream reaches the call.
 *   - Arguments are validated on the host before anything is launched; a
 *     nonzero status launches nothing and leaves outputs untouched.  A short
 *     message for the last failure on the calling thread is in sv_last_error().
 *   - Inputs must be finite (sv_accept_sample also takes -inf logits, see there).
 *     Results are bitwise reproducible for identical inputs and shapes.
 *   - Workspaces carry no state between calls and need no initialisation; two
 *     calls that share one workspace must not overlap in time.
 *   - Inside sv_accept_sample and sv_accept_sample_tree, some workgroups wait for
 *     results that other workgroups of the same launch publish (agent-scope atomic
 *     stores and loads, no fences): the last race workgroup of each sequence, and the
 *     residual passes of a tree run as one launch when the device holds those
 *     workgroups at once.  A race workgroup waits only on workgroups that in-order
 *     dispatch started before it; a tree pass waits only on workgroups that are
 *     resident with it.  Every wait is bounded besides (sv_set_wait_limit), so a launch
 *     always ends; a sequence whose wait gave up (only if other work held the device
 *     for a large fraction of a second) reports accept_len -1 and out_tokens (and
 *     accept_path) all -1.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_API_VERSION 1

typedef enum { SV_F32 = 0, SV_BF16 = 1, SV_F16 = 2 } sv_dtype;

typedef enum {
  SV_OK = 0,
  SV_ERR_INVALID_ARG = -1, /* a shape, pointer or value is out of its documented range */
  SV_ERR_UNSUPPORTED = -2, /* a valid request this build does not implement (dtype, head_dim) */
  SV_ERR_WORKSPACE = -3,   /* workspace pointer NULL or smaller than the size query says */
  SV_ERR_DEVICE = -4       /* the HIP runtime refused a launch */
} sv_status;

int sv_version(void);
const char* sv_status_string(int status);
/* Message of the last failed call on this thread ("" if none). */
const char* sv_last_error(void);
/* Polls a waiting workgroup of sv_accept_sample / sv_accept_sample_tree makes before it
 * gives up and reports its sequence as failed (accept_len -1, see the conventions
 * above): polls >= 1, default 262,144 (2^18), process-wide, read by each call when it
 * launches.  For callers that prefer an early, reported failure to a long wait, and for
 * tests of that path (a small limit makes the waits give up without any fault).
 * SV_ERR_INVALID_ARG for polls < 1. */
sv_status sv_set_wait_limit(int32_t polls);

/* -------------------------------------------------------------------------------------
 * Block-verification attention.
 *
 * Operation (VFlash-FM page, "How VFlash-FM works": the target scores all K block
 * positions in one forward over the full context; demo setup: native grouped-query
 * attention, preallocated KV caches).  For sequence b, block row i in [0, K) and
 * query head h, with G = Hq / Hkv and KV head g = h / G:
 *     visible keys: context positions 0 .. ctx_lens[b]-1, plus block position
 *                   ctx_lens[b] + t whenever bit t of block_mask[i] is set;
 *     s_j = scale * <q[b][i][h], k_j>,  out[b][i][h] = sum_j softmax(s)_j v_j,
 *     lse[b][i][h] = log sum_j exp(s_j)  (natural log).
 *
 * Layouts
 *   q          [B][K][Hq][d]               dtype
 *   k_cache    [num_pages][Hkv][P][d]      dtype, token-major pages
 *   v_cache    [num_pages][Hkv][d][P]      dtype, dim-major pages (each head's page is
 *                                          d rows of P consecutive tokens)
 *   page_table [B][max_pages_per_seq]      int32: token j of sequence b lives in page
 *                                          page_table[b][j / P], slot j % P
 *   ctx_lens   [B]                         int32: context tokens before the block; the
 *                                          block's own K/V rows are already written at
 *                                          positions ctx .. ctx+K-1 (see sv_kv_append)
 *   block_mask HOST [K] uint64             row masks over the block keys; NULL = causal
 *                                          (bit t of row i set iff t <= i)
 *   out        [B][K][Hq][d]               dtype (round to nearest even from fp32)
 *   lse        [B][K][Hq]                  fp32, optional (NULL = not written)
 *
 * Limits: 1 <= K <= 64; Hq % Hkv == 0; K * G <= 512; d in {64, 128}; P a power of two
 * in [16, 256]; every block_mask row i must contain bit i and no bit >= K.
 * ctx_lens[b] must lie in [0, max_ctx] and ctx_lens[b] + K <= max_pages_per_seq * P.
 * Device-side, keys beyond max_ctx + K and table entries outside [0, num_pages) are
 * never dereferenced (their K/V read as zero), so a violation gives wrong numbers,
 * never an out-of-bounds access.
 * ------------------------------------------------------------------------------------ */
typedef struct {
  int32_t batch;             /* B >= 1 */
  int32_t block;             /* K */
  int32_t num_q_heads;       /* Hq */
  int32_t num_kv_heads;      /* Hkv */
  int32_t head_dim;          /* d */
  int32_t page_size;         /* P */
  int32_t max_pages_per_seq; /* row stride of page_table */
  int32_t num_pages;         /* pages in the pool (for device-side bounds) */
  int32_t max_ctx;           /* host-known upper bound of ctx_lens: sizes the split grid */
  int32_t split_keys;        /* keys per split-KV work item; 0 = automatic, else a
                                multiple of min(page_size, 64), at most 16384 */
  float scale;               /* 0 => 1/sqrt(d) */
  sv_dtype dtype;            /* q, caches and out */
  int64_t sum_ctx_hint;      /* host-known sum of ctx_lens, steers the automatic split
                                size only; 0 = unknown (taken as B * max_ctx) */
} sv_attn_desc;

/* Bytes of workspace sv_verify_attention needs for this descriptor. */
sv_status sv_verify_attention_workspace(const sv_attn_desc* desc, size_t* bytes);

sv_status sv_verify_attention(const sv_attn_desc* desc, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* page_table,
                              const int32_t* ctx_lens, const uint64_t* block_mask, void* out,
                              float* lse, void* workspace, size_t workspace_bytes,
                              void* stream);

/* -------------------------------------------------------------------------------------
 * Allocation-free verify attention, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same operation, arguments, layouts, limits and results as sv_verify_attention, without
 * the workspace arguments: the split-KV partials go to a scratch array of
 * SV_NOALLOC_SCRATCH_BYTES held by the library on each GPU it runs on (until the process
 * ends).  Descriptors whose sv_verify_attention_workspace exceeds that size are rejected
 * with SV_ERR_WORKSPACE.  The call allocates, frees and clears nothing; it runs on the
 * current device, and `stream` must belong to it (else SV_ERR_INVALID_ARG).  All calls on
 * one GPU share its scratch array: calls that overlap in time on one GPU (several streams
 * or host threads) race and give wrong results.
 * ------------------------------------------------------------------------------------ */
#define SV_NOALLOC_SCRATCH_BYTES (32u << 20)

sv_status sv_verify_attention_noalloc(const sv_attn_desc* desc, const void* q,
                                      const void* k_cache, const void* v_cache,
                                      const int32_t* page_table, const int32_t* ctx_lens,
                                      const uint64_t* block_mask, void* out, float* lse,
                                      void* stream);

/* -------------------------------------------------------------------------------------
 * Greedy acceptance (VFlash-FM page, caption of the cycle figure: the prefix matching
 * the target's greedy choice is accepted, the target supplies the token at the first
 * disagreement, the rest is discarded).
 *   t_i = argmax_j logits[b][i][j], ties to the lowest j  (i = 0 .. K-1)
 *   accept_len[b] = largest a <= K-1 with drafts[b][k-1] == t_{k-1} for all k <= a
 *   out_tokens[b] = drafts[b][0 .. a-1], t_a, then -1 up to K entries
 *   argmax[b][i]  = t_i (optional, NULL = not written)
 * Layouts: logits [B][K][V] (SV_F32 or SV_BF16); drafts [B][K-1] int32 (draft d_k at
 * index k-1); accept_len [B], out_tokens [B][K], argmax [B][K] int32.
 * Limits: 1 <= K <= 64, 1 <= V < 2^31.  Workspace: B*K*32 packed keys (no initial state).
 * ------------------------------------------------------------------------------------ */
sv_status sv_accept_greedy_workspace(int32_t B, int32_t K, int32_t V, size_t* bytes);
sv_status sv_accept_greedy(int32_t B, int32_t K, int32_t V, sv_dtype logit_dtype,
                           const void* logits, const int32_t* drafts, int32_t* accept_len,
                           int32_t* out_tokens, int32_t* argmax, void* workspace,
                           size_t workspace_bytes, void* stream);

/* -------------------------------------------------------------------------------------
 * Sampling acceptance: the standard speculative acceptance-rejection rule (SpecFLASH
 * README, "components": drafts verified in parallel by the target with the standard
 * rule, so the output follows the target's distribution exactly).
 *   p_i = softmax(target_logits[b][i] / T), q_k = softmax(draft_logits[b][k-1] / T)
 *   for k = 1 .. K-1: accept d_k iff u_k < min(1, p_{k-1}(d_k) / q_k(d_k));
 *   first rejection at k: resample from norm(max(0, p_{k-1} - q_k));
 *   all accepted: bonus token from p_{K-1}.
 * Uniforms: Philox4x64-10 with key (seed, 0), counter (offset, b, (purpose << 32) | row,
 * j >> 2), word j & 3, u = (word >> 11) * 2^-53; purpose 0 (accept test, row = k, j = 0),
 * purpose 1 (resample, row = target row raced over, j = token).  The resample draws
 * argmin_j E_j / r_j with E_j = -ln(1 - u_j) over r_j > 0 (an exponential race, exact
 * in distribution), ties to the lowest j.  The ratio test and the race run in fp64; the
 * row log-normalisers use fp32 exponentials summed in fp64.
 * Layouts: target_logits [B][K][V], draft_logits [B][K-1][V] (SV_F32 or SV_BF16), both
 * 16-byte aligned; drafts [B][K-1] int32; outputs as for sv_accept_greedy.  A draft
 * outside [0, V) counts as rejected (its logits are never read).
 * Logits may be -inf: such an entry has probability 0 (a masked vocabulary).  A draft
 * whose target probability is 0 is always rejected; one whose draft probability is 0
 * (but target probability is not) is always accepted.  Every row must hold at least
 * one finite logit; +inf and NaN are not supported.  A draw over a row without any
 * finite logit has nothing to draw from and is reported as token -1.
 * Limits: 2 <= K <= 64, 1 <= V < 2^31, B * (2K - 1) <= 65535, temperature > 0 (greedy is
 * its own call).  The workspace (16-byte aligned) needs no initial contents.
 * ------------------------------------------------------------------------------------ */
sv_status sv_accept_sample_workspace(int32_t B, int32_t K, int32_t V, size_t* bytes);
sv_status sv_accept_sample(int32_t B, int32_t K, int32_t V, sv_dtype logit_dtype,
                           const void* target_logits, const void* draft_logits,
                           const int32_t* drafts, float temperature, uint64_t seed,
                           uint64_t offset, int32_t* accept_len, int32_t* out_tokens,
                           void* workspace, size_t workspace_bytes, void* stream);

/* -------------------------------------------------------------------------------------
 * Latent visual compressor (SpecFLASH README, "components", compressor equation):
 *   out[b] = softmax(scale * queries . feats[b]^T) . feats[b], softmax over the N rows.
 * The printed formula has no 1/sqrt(D); pass scale = 1 for it (0 is read as 1).
 * Layouts: queries [C][D], feats [B][N][D], out [B][C][D], all SV_F16 (fp32 accumulate),
 * each 16-byte aligned, as is the workspace (no initial contents).
 * Limits: 1 <= C <= 64, 1 <= N <= 1024, D a multiple of 128 (invalid: SV_ERR_INVALID_ARG).
 * ------------------------------------------------------------------------------------ */
sv_status sv_latent_compress_workspace(int32_t B, int32_t C, int32_t N, int32_t D,
                                       size_t* bytes);
sv_status sv_latent_compress(int32_t B, int32_t C, int32_t N, int32_t D, sv_dtype dtype,
                             const void* queries, const void* feats, void* out, float scale,
                             void* workspace, size_t workspace_bytes, void* stream);

/* -------------------------------------------------------------------------------------
 * KV append: write n new token rows per sequence into the paged cache at positions
 * start[b] .. start[b]+n-1 (the preallocated KV cache the VFlash-FM demo setup names;
 * the block's rows must be in place before sv_verify_attention).
 *   k_new, v_new [B][n][Hkv][d] (token-major rows, dtype of the cache); start [B] int32.
 * Uses desc->batch, num_kv_heads, head_dim, page_size, max_pages_per_seq, num_pages,
 * dtype.  Positions must satisfy start[b] + n <= max_pages_per_seq * P; rows whose
 * page-table entry is outside [0, num_pages) are skipped.  No workspace.
 * ------------------------------------------------------------------------------------ */
sv_status sv_kv_append(const sv_attn_desc* desc, int32_t n, const void* k_new,
                       const void* v_new, const int32_t* start, const int32_t* page_table,
                       void* k_cache, void* v_cache, void* stream);

/* -------------------------------------------------------------------------------------
 * Cycle commit (VFlash-FM page, caption of the cycle figure: the accepted drafts and
 * the target's token at the first disagreement are committed, and that token anchors
 * the next cycle).  Per sequence b, with a = accept_len[b] (clamped to [0, K-1]):
 *   next_anchor[b] = out_tokens[b][a];   ctx_lens[b] += a + 1
 * -- the anchor and the a accepted drafts keep the K/V rows written before the verify
 * pass; rejected drafts' rows are overwritten by the next block's sv_kv_append, so no
 * rollback is needed.  accept_len [B], out_tokens [B][K] are the outputs of
 * sv_accept_greedy / sv_accept_sample; ctx_lens [B] is updated in place; next_anchor
 * [B] int32 is written.  All device pointers; no workspace.  The caller keeps
 * ctx_lens[b] + K within max_pages_per_seq * page_size for the next cycle.
 * ------------------------------------------------------------------------------------ */
sv_status sv_commit(int32_t B, int32_t K, const int32_t* accept_len, const int32_t* out_tokens,
                    int32_t* ctx_lens, int32_t* next_anchor, void* stream);

/* -------------------------------------------------------------------------------------
 * Draft trees (the tree-verified "Tree-60" variant of the VFlash-FM results table).
 * Node 0 is the anchor (block row 0); nodes 1 .. K-1 carry the drafts, and a parent has
 * a smaller number than its children.  The block is appended in node order and verified
 * with sv_verify_attention using the tree's mask rows (row i: bit j set iff node j is
 * node i or an ancestor of it), so row i is the target's prediction after node i.
 *
 * Greedy tree acceptance: the chain rule walked from the anchor.  At the current node,
 * the child (numbered above it) whose token equals the target's greedy token of the
 * current node's row is accepted and becomes the current node -- the lowest-numbered
 * one if several siblings share that token; the walk stops at the first node with no
 * such child, whose greedy token is the correction.
 *   logits [B][K][V] (SV_F32 or SV_BF16); parents [B][K-1], tokens [B][K-1] int32:
 *   parent and draft token of node i at [b][i-1].
 *   accept_len [B]: accepted depth a; out_tokens [B][K]: the accepted nodes' tokens, then
 *   the correction, then -1; accept_path [B][K]: 0, the accepted nodes, then -1;
 *   argmax [B][K] optional.  Workspace: sv_accept_greedy_workspace(B, K, V) bytes.
 * A parent array that is not a tree (parent >= node) never makes the walk leave [0, K)
 * or run more than K-1 steps; such nodes are simply never reached.
 * Limits as for sv_accept_greedy.
 * ------------------------------------------------------------------------------------ */
sv_status sv_accept_greedy_tree(int32_t B, int32_t K, int32_t V, sv_dtype logit_dtype,
                                const void* logits, const int32_t* parents,
                                const int32_t* tokens, int32_t* accept_len,
                                int32_t* out_tokens, int32_t* accept_path, int32_t* argmax,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Sampling verification of a draft tree: the standard acceptance-rejection rule (SpecFLASH
 * README, "components") applied as recursive rejection over the children of the current
 * node, for the tree-verified variant of the VFlash-FM results table.  At node u (target
 * row u, p_u = softmax(row / T)) the children c_1 < c_2 < ... are tested in order; child
 * c_j, token x_j drawn from q_j = softmax(draft row of c_j / T), passes iff
 * u_j < min(1, r_{j-1}(x_j) / q_j(x_j)), with r_0 = p_u and, after each rejection,
 * r_j = norm(max(0, r_{j-1} - q_j)) (p_u if that is all zero).  The first child that
 * passes becomes the current node; when none does (or u is a leaf) the token is drawn
 * from the last residual by the exponential race.  Uniforms as for sv_accept_sample: the
 * test of node c uses purpose 0 with row c, the draw purpose 1 with the row of the node
 * the walk stopped at; on a chain the call returns exactly what sv_accept_sample returns.
 *   target_logits [B][K][V], draft_logits [B][K-1][V] (row i-1: the distribution node i was
 *   drawn from; siblings may share one or differ), SV_F32 or SV_BF16, 16-byte aligned;
 *   parents HOST [K-1] int32, the tree shared by the batch (parent of node i at [i-1], in
 *   [0, i): checked, else SV_ERR_INVALID_ARG); tokens [B][K-1] device int32 (a token
 *   outside [0, V) is rejected).  Outputs as for sv_accept_greedy_tree: accept_len [B],
 *   out_tokens [B][K] (accepted nodes' tokens, the drawn token, then -1), accept_path
 *   [B][K] (0, the accepted nodes, then -1); close the cycle with sv_commit_tree.
 * -inf logits are probability 0 as for sv_accept_sample.  Limits: 2 <= K <= 64,
 * B * (2K - 1) <= 65535, T > 0.  Workspace: sv_accept_sample_tree_workspace bytes, 16-byte
 * aligned, no initial contents.  The tree's largest child count m sets m - 1 sequential
 * residual passes over the vocabulary (none on a chain).
 * ------------------------------------------------------------------------------------ */
sv_status sv_accept_sample_tree_workspace(int32_t B, int32_t K, int32_t V, size_t* bytes);
sv_status sv_accept_sample_tree(int32_t B, int32_t K, int32_t V, sv_dtype logit_dtype,
                                const void* target_logits, const void* draft_logits,
                                const int32_t* parents, const int32_t* tokens, float temperature,
                                uint64_t seed, uint64_t offset, int32_t* accept_len,
                                int32_t* out_tokens, int32_t* accept_path, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Tree commit: per sequence b with a = accept_len[b] (clamped to [0, K-1]) and
 * K = desc->block, the K/V rows of the j-th accepted node move from position
 * ctx + accept_path[b][j] to ctx + j (j = 1 .. a; every source is read before any
 * destination is written), then as sv_commit: next_anchor[b] = out_tokens[b][a] and
 * ctx_lens[b] += a + 1.  desc gives B, K, Hkv, d, P, the table stride, the pool size and
 * the dtype of the caches (laid out as for sv_verify_attention).  Sequences whose
 * ctx_lens[b] + K exceeds the page table, and table entries outside [0, num_pages), move
 * nothing.  All device pointers; no workspace.
 * ------------------------------------------------------------------------------------ */
sv_status sv_commit_tree(const sv_attn_desc* desc, const int32_t* accept_len,
                         const int32_t* out_tokens, const int32_t* accept_path,
                         const int32_t* page_table, void* k_cache, void* v_cache,
                         int32_t* ctx_lens, int32_t* next_anchor, void* stream);

/* -------------------------------------------------------------------------------------
 * LM head fused with greedy acceptance (the last step of the verify forward, then the
 * greedy rule of the VFlash-FM cycle figure): logits[b][i][v] = <hidden_states[b][i],
 * weight[v]> accumulated in fp32, never written to memory; t_i = the lowest-index argmax
 * of row i; then the chain rule exactly as sv_accept_greedy (same outputs).
 * Layouts: hidden_states [B][K][hidden], weight [V][hidden] (the output embedding, row
 * per token), both SV_BF16 or SV_F16; drafts [B][K-1].  The weight is read once.
 * Limits: B * K <= 64, hidden a multiple of 32, 1 <= V < 2^31, 1 <= K <= 64.
 * Workspace: sv_lm_head_greedy_workspace bytes, 8-byte aligned, no initial contents.
 * ------------------------------------------------------------------------------------ */
sv_status sv_lm_head_greedy_workspace(int32_t B, int32_t K, int32_t V, int32_t hidden,
                                      size_t* bytes);
sv_status sv_lm_head_greedy(int32_t B, int32_t K, int32_t V, int32_t hidden, sv_dtype dtype,
                            const void* hidden_states, const void* weight,
                            const int32_t* drafts, int32_t* accept_len, int32_t* out_tokens,
                            int32_t* argmax, void* workspace, size_t workspace_bytes,
                            void* stream);

/* -------------------------------------------------------------------------------------
 * The same LM head over a pre-packed weight.  The output embedding does not change
 * between cycles, so it can be rearranged once, when it is loaded, into the order in
 * which the argmax pass consumes it: every load instruction then reads one contiguous
 * kilobyte and the stream is read with non-temporal loads.
 * sv_lm_head_pack_bytes: the packed size, ceil(V / 32) * 32 * hidden * 2 bytes.
 * sv_lm_head_pack: weight [V][hidden] (SV_BF16 or SV_F16) -> packed, in the tile layout:
 *   tiles of 16 rows x 32 columns; tile (u, q, h) covers rows 32u + 16h .. 32u + 16h + 15
 *   and columns 32q .. 32q + 31, its 16-byte piece 16g + j holding row 32u + 16h + j,
 *   columns 32q + 8g .. 32q + 8g + 7; tiles stored in the order u, q, h; rows at or past V
 *   are zero.  Both device pointers, 16-byte aligned, not overlapping; V >= 1, hidden a
 *   positive multiple of 32.  Enqueued on stream; no workspace.
 * sv_lm_head_greedy_packed: exactly sv_lm_head_greedy (same arguments, limits, workspace
 *   and outputs, bit for bit) with packed_weight = the output of sv_lm_head_pack for the
 *   same V, hidden and dtype in place of weight.
 * ------------------------------------------------------------------------------------ */
sv_status sv_lm_head_pack_bytes(int32_t V, int32_t hidden, size_t* bytes);
sv_status sv_lm_head_pack(int32_t V, int32_t hidden, sv_dtype dtype, const void* weight,
                          void* packed, void* stream);
sv_status sv_lm_head_greedy_packed(int32_t B, int32_t K, int32_t V, int32_t hidden,
                                   sv_dtype dtype, const void* hidden_states,
                                   const void* packed_weight, const int32_t* drafts,
                                   int32_t* accept_len, int32_t* out_tokens, int32_t* argmax,
                                   void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SPECVERIFY_H */
