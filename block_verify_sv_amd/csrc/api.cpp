// libspecverify C ABI: argument validation, work planning and launches.
// Every check runs on the host before anything touches the GPU, so invalid calls fail
// with a status code (and a message in sv_last_error) and launch nothing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>
#include <atomic>
#include <string>

#include "internal.hpp"
#include "specverify.h"

namespace {

thread_local std::string g_last_error;

sv_status fail(sv_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
sv_status fail(sv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

sv_status ok() {
  g_last_error.clear();
  return SV_OK;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// The value a caller stored in an sv_dtype, read as its bytes: a C caller may pass any int,
// and C++ may only load an enum value in the enumerators' range, so every check reads this.
int32_t dtype_bits(const sv_dtype* p) {
  int32_t v;
  memcpy(&v, p, sizeof v);
  return v;
}

bool dtype_in(int32_t v, std::initializer_list<sv_dtype> ok) {
  for (sv_dtype d : ok)
    if (v == static_cast<int32_t>(d)) return true;
  return false;
}

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

sv_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SV_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// ---------------------------------------------------------------- attention checks
sv_status check_attn_desc(const sv_attn_desc* d) {
  if (!d) return fail(SV_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch < 1 || d->batch > 65535)
    return fail(SV_ERR_INVALID_ARG, "batch must be in [1, 65535] (got %d)", d->batch);
  if (d->block < 1 || d->block > sv::kMaxBlock)
    return fail(SV_ERR_INVALID_ARG, "block must be in [1, 64] (got %d)", d->block);
  if (d->num_q_heads < 1 || d->num_kv_heads < 1 || d->num_q_heads > 65535)
    return fail(SV_ERR_INVALID_ARG, "head counts must be in [1, 65535]");
  if (d->num_q_heads % d->num_kv_heads != 0)
    return fail(SV_ERR_INVALID_ARG, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)",
                d->num_q_heads, d->num_kv_heads);
  const int G = d->num_q_heads / d->num_kv_heads;
  if (d->block * G > sv::kMaxRows)
    return fail(SV_ERR_INVALID_ARG, "block * (num_q_heads / num_kv_heads) = %d exceeds %d",
                d->block * G, sv::kMaxRows);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(SV_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", d->head_dim);
  if (!dtype_in(dtype_bits(&d->dtype), {SV_F32, SV_BF16, SV_F16}))
    return fail(SV_ERR_UNSUPPORTED, "unknown dtype %d", dtype_bits(&d->dtype));
  if (!pow2(d->page_size) || d->page_size < 16 || d->page_size > 256)
    return fail(SV_ERR_INVALID_ARG, "page_size must be a power of two in [16, 256] (got %d)",
                d->page_size);
  if (d->max_pages_per_seq < 1 || d->num_pages < 1)
    return fail(SV_ERR_INVALID_ARG, "max_pages_per_seq and num_pages must be >= 1");
  if (d->max_ctx < 0) return fail(SV_ERR_INVALID_ARG, "max_ctx must be >= 0");
  if (static_cast<int64_t>(d->max_ctx) + d->block >
      static_cast<int64_t>(d->max_pages_per_seq) * d->page_size)
    return fail(SV_ERR_INVALID_ARG,
                "max_ctx + block (%lld) exceeds max_pages_per_seq * page_size (%lld)",
                static_cast<long long>(d->max_ctx) + d->block,
                static_cast<long long>(d->max_pages_per_seq) * d->page_size);
  if (static_cast<int64_t>(d->max_ctx) + d->block > (1ll << 30))
    return fail(SV_ERR_INVALID_ARG, "max_ctx too large");
  const int gran = d->page_size < 64 ? d->page_size : 64;
  if (d->split_keys < 0 || (d->split_keys % gran) != 0 || d->split_keys > sv::kMaxSplitKeys)
    return fail(SV_ERR_INVALID_ARG,
                "split_keys must be 0 or a multiple of min(page_size, 64) = %d, at most 16384 "
                "(got %d)", gran, d->split_keys);
  if (!(d->scale >= 0.0f) || !isfinite(d->scale))
    return fail(SV_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if (d->sum_ctx_hint < 0) return fail(SV_ERR_INVALID_ARG, "sum_ctx_hint must be >= 0");
  return SV_OK;
}

}  // namespace


namespace sv {
namespace {
std::atomic<int32_t> g_wait_limit{1 << 18};
}  // namespace
int32_t wait_limit() { return g_wait_limit.load(std::memory_order_relaxed); }
}  // namespace sv

extern "C" {

int sv_version(void) { return SV_API_VERSION; }

const char* sv_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_INVALID_ARG: return "invalid argument";
    case SV_ERR_UNSUPPORTED: return "unsupported";
    case SV_ERR_WORKSPACE: return "workspace too small";
    case SV_ERR_DEVICE: return "device error";
    default: return "unknown status";
  }
}

const char* sv_last_error(void) { return g_last_error.c_str(); }

sv_status sv_set_wait_limit(int32_t polls) {
  if (polls < 1) return fail(SV_ERR_INVALID_ARG, "sv_set_wait_limit: polls must be >= 1");
  sv::g_wait_limit.store(polls, std::memory_order_relaxed);
  return SV_OK;
}

// ---------------------------------------------------------------- attention
sv_status sv_verify_attention_workspace(const sv_attn_desc* desc, size_t* bytes) {
  sv_status st = check_attn_desc(desc);
  if (st != SV_OK) return st;
  if (!bytes) return fail(SV_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = sv::plan_attention(*desc).ws_bytes;
  return ok();
}

sv_status sv_verify_attention(const sv_attn_desc* desc, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* page_table,
                              const int32_t* ctx_lens, const uint64_t* block_mask, void* out,
                              float* lse, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return sv::attention_call(desc, q, k_cache, v_cache, page_table, ctx_lens, block_mask, out, lse,
                            workspace, workspace_bytes, stream, "sv_verify_attention launch");
}

}  // extern "C"

namespace sv {

sv_status report(sv_status st, const char* msg) {
  if (st == SV_OK) return ok();
  return fail(st, "%s", msg);
}

sv_status attention_call(const sv_attn_desc* desc, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* page_table, const int32_t* ctx_lens,
                         const uint64_t* block_mask, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream, const char* what) {
  sv_status st = check_attn_desc(desc);
  if (st != SV_OK) return st;
  if (!q || !k_cache || !v_cache || !page_table || !ctx_lens || !out)
    return fail(SV_ERR_INVALID_ARG, "q, k_cache, v_cache, page_table, ctx_lens and out are required");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(SV_ERR_INVALID_ARG, "q, k_cache, v_cache and out must be 16-byte aligned");
  const int K = desc->block;
  sv::AttnParams p;
  memset(&p, 0, sizeof p);
  for (int i = 0; i < K; ++i) {
    const uint64_t m = block_mask ? block_mask[i] : ((i == 63) ? ~0ull : ((1ull << (i + 1)) - 1));
    if (!((m >> i) & 1ull))
      return fail(SV_ERR_INVALID_ARG, "block_mask row %d must contain its own bit", i);
    if (K < 64 && (m >> K) != 0)
      return fail(SV_ERR_INVALID_ARG, "block_mask row %d has bits at or beyond block %d", i, K);
    p.mask[i] = m;
  }
  const sv::AttnPlan pl = sv::plan_attention(*desc);
  if (!workspace || workspace_bytes < pl.ws_bytes)
    return fail(SV_ERR_WORKSPACE, "attention needs %zu workspace bytes (got %zu)", pl.ws_bytes,
                workspace ? workspace_bytes : 0);
  if (!aligned16(workspace)) return fail(SV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.page_table = page_table;
  p.ctx_lens = ctx_lens;
  p.part_o = workspace;
  p.part_ml = reinterpret_cast<float2*>(static_cast<char*>(workspace) + pl.o_bytes);
  p.out = out;
  p.lse = lse;
  p.B = desc->batch;
  p.K = K;
  p.Hq = desc->num_q_heads;
  p.Hkv = desc->num_kv_heads;
  p.G = desc->num_q_heads / desc->num_kv_heads;
  p.R = pl.rows;
  p.P_log2 = log2i(desc->page_size);
  p.max_pages = desc->max_pages_per_seq;
  p.num_pages = desc->num_pages;
  p.max_ctx = desc->max_ctx;
  p.chunk = pl.chunk;
  p.nsplit = pl.nsplit;
  // a multiple of 8 keeps split s of every head on one XCD (measured 1-2% faster on the
  // 7B and batched workloads) and lets row groups share an XCD; below 8 splits with one
  // row group the padding would mostly add empty workgroups (8x for a single split)
  p.nsplit_pad = (pl.row_groups > 1 || pl.nsplit >= 8) ? (pl.nsplit + 7) / 8 * 8 : pl.nsplit;
  p.direct = pl.nsplit == 1 ? 1 : 0;
  p.row_groups = pl.row_groups;
  const float scale = desc->scale > 0.0f ? desc->scale : 1.0f / sqrtf(static_cast<float>(desc->head_dim));
  p.scale_log2 = scale * 1.4426950408889634f;
  return device_status(sv::launch_attention(p, desc->head_dim, desc->dtype,
                                            static_cast<hipStream_t>(stream)),
                       what);
}

}  // namespace sv

extern "C" {

// ---------------------------------------------------------------- greedy
static sv_status check_accept_shape(int32_t B, int32_t K, int32_t V, int min_k) {
  if (B < 1) return fail(SV_ERR_INVALID_ARG, "B must be >= 1 (got %d)", B);
  if (K < min_k || K > sv::kMaxBlock)
    return fail(SV_ERR_INVALID_ARG, "K must be in [%d, 64] (got %d)", min_k, K);
  if (V < 1) return fail(SV_ERR_INVALID_ARG, "V must be >= 1 (got %d)", V);
  if (static_cast<int64_t>(B) * K > 65535)
    return fail(SV_ERR_INVALID_ARG, "B * K must be <= 65535 (got %lld)",
                static_cast<long long>(B) * K);
  return SV_OK;
}

sv_status sv_accept_greedy_workspace(int32_t B, int32_t K, int32_t V, size_t* bytes) {
  sv_status st = check_accept_shape(B, K, V, 1);
  if (st != SV_OK) return st;
  if (!bytes) return fail(SV_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = sv::greedy_workspace_bytes(B, K);
  return ok();
}

// The chain (parents == nullptr) and the tree walk share the argmax pass.
static sv_status greedy_call(int32_t B, int32_t K, int32_t V, int32_t dtype_raw,
                             const void* logits, const int32_t* drafts, const int32_t* parents,
                             int32_t* path, int32_t* accept_len, int32_t* out_tokens,
                             int32_t* argmax, void* workspace, size_t workspace_bytes,
                             void* stream, const char* what) {
  sv_status st = check_accept_shape(B, K, V, 1);
  if (st != SV_OK) return st;
  if (!dtype_in(dtype_raw, {SV_F32, SV_BF16}))
    return fail(SV_ERR_UNSUPPORTED, "greedy logits must be SV_F32 or SV_BF16");
  const sv_dtype logit_dtype = static_cast<sv_dtype>(dtype_raw);
  if (!logits || !accept_len || !out_tokens || (K > 1 && !drafts))
    return fail(SV_ERR_INVALID_ARG, "logits, drafts, accept_len and out_tokens are required");
  if (!aligned16(logits)) return fail(SV_ERR_INVALID_ARG, "logits must be 16-byte aligned");
  const size_t need = sv::greedy_workspace_bytes(B, K);
  if (!workspace || workspace_bytes < need)
    return fail(SV_ERR_WORKSPACE, "greedy accept needs %zu workspace bytes", need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 7u) != 0)
    return fail(SV_ERR_INVALID_ARG, "workspace must be 8-byte aligned");
  sv::GreedyParams p;
  p.logits = logits;
  p.drafts = drafts;
  p.parents = parents;
  p.path = path;
  p.tree = path != nullptr;
  p.accept_len = accept_len;
  p.out_tokens = out_tokens;
  p.argmax = argmax;
  p.keys = static_cast<unsigned long long*>(workspace);
  p.B = B;
  p.K = K;
  p.V = V;
  p.chunk = sv::greedy_chunk(V, logit_dtype);
  p.nchunk = (V + p.chunk - 1) / p.chunk;
  if (static_cast<int64_t>(p.nchunk) * K >= (1ll << 31))
    return fail(SV_ERR_INVALID_ARG, "V too large");
  return device_status(sv::launch_greedy(p, logit_dtype, static_cast<hipStream_t>(stream)), what);
}

sv_status sv_accept_greedy(int32_t B, int32_t K, int32_t V, sv_dtype logit_dtype,
                           const void* logits, const int32_t* drafts, int32_t* accept_len,
                           int32_t* out_tokens, int32_t* argmax, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return greedy_call(B, K, V, dtype_bits(&logit_dtype), logits, drafts, nullptr, nullptr, accept_len,
                     out_tokens, argmax, workspace, workspace_bytes, stream,
                     "sv_accept_greedy launch");
}

sv_status sv_accept_greedy_tree(int32_t B, int32_t K, int32_t V, sv_dtype logit_dtype,
                                const void* logits, const int32_t* parents,
                                const int32_t* tokens, int32_t* accept_len,
                                int32_t* out_tokens, int32_t* accept_path, int32_t* argmax,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (K > 1 && !parents) return fail(SV_ERR_INVALID_ARG, "parents is required");
  if (!accept_path) return fail(SV_ERR_INVALID_ARG, "accept_path is required");
  return greedy_call(B, K, V, dtype_bits(&logit_dtype), logits, tokens, parents, accept_path, accept_len,
                     out_tokens, argmax, workspace, workspace_bytes, stream,
                     "sv_accept_greedy_tree launch");
}

// ---------------------------------------------------------------- LM head + greedy
static sv_status check_lm_head(int32_t B, int32_t K, int32_t V, int32_t hidden) {
  sv_status st = check_accept_shape(B, K, V, 1);
  if (st != SV_OK) return st;
  if (static_cast<int64_t>(B) * K > 64)
    return fail(SV_ERR_INVALID_ARG, "B * K must be <= 64 (got %lld)", static_cast<long long>(B) * K);
  if (hidden < 32 || hidden % 32 != 0 || hidden > (1 << 20))
    return fail(SV_ERR_INVALID_ARG, "hidden must be a positive multiple of 32 (got %d)", hidden);
  return SV_OK;
}

sv_status sv_lm_head_greedy_workspace(int32_t B, int32_t K, int32_t V, int32_t hidden,
                                      size_t* bytes) {
  sv_status st = check_lm_head(B, K, V, hidden);
  if (st != SV_OK) return st;
  if (!bytes) return fail(SV_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = sv::lm_head_workspace_bytes(B * K, V);
  return ok();
}

// dtype arrives as its raw bits: a C caller may pass any int, which is not a valid
// sv_dtype value until checked.
static sv_status lm_head_call(int32_t B, int32_t K, int32_t V, int32_t hidden, int32_t dtype,
                              const void* hidden_states, const void* weight, bool packed,
                              const int32_t* drafts, int32_t* accept_len, int32_t* out_tokens,
                              int32_t* argmax, void* workspace, size_t workspace_bytes,
                              void* stream, const char* what) {
  sv_status st = check_lm_head(B, K, V, hidden);
  if (st != SV_OK) return st;
  if (!dtype_in(dtype, {SV_BF16, SV_F16}))
    return fail(SV_ERR_UNSUPPORTED, "LM head operands must be SV_BF16 or SV_F16");
  if (!hidden_states || !weight || !accept_len || !out_tokens || (K > 1 && !drafts))
    return fail(SV_ERR_INVALID_ARG, "hidden_states, weight, drafts and outputs are required");
  if (!aligned16(hidden_states) || !aligned16(weight))
    return fail(SV_ERR_INVALID_ARG, "hidden_states and weight must be 16-byte aligned");
  const int M = B * K;
  const size_t need = sv::lm_head_workspace_bytes(M, V);
  if (!workspace || workspace_bytes < need)
    return fail(SV_ERR_WORKSPACE, "LM head needs %zu workspace bytes", need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 7u) != 0)
    return fail(SV_ERR_INVALID_ARG, "workspace must be 8-byte aligned");
  sv::LmHeadParams p;
  p.hidden = hidden_states;
  p.weight = weight;
  p.nwg = 0;
  p.part = static_cast<unsigned long long*>(workspace);
  p.M = M;
  p.V = V;
  p.Hd = hidden;
  p.packed = packed ? 1 : 0;
  sv::GreedyParams w;
  memset(&w, 0, sizeof w);
  w.drafts = drafts;
  w.accept_len = accept_len;
  w.out_tokens = out_tokens;
  w.argmax = argmax;
  w.B = B;
  w.K = K;
  w.V = V;
  return device_status(sv::launch_lm_head(p, w, static_cast<sv_dtype>(dtype),
                                          static_cast<hipStream_t>(stream)), what);
}

sv_status sv_lm_head_greedy(int32_t B, int32_t K, int32_t V, int32_t hidden, sv_dtype dtype,
                            const void* hidden_states, const void* weight,
                            const int32_t* drafts, int32_t* accept_len, int32_t* out_tokens,
                            int32_t* argmax, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return lm_head_call(B, K, V, hidden, dtype_bits(&dtype), hidden_states, weight, false, drafts,
                      accept_len, out_tokens, argmax, workspace, workspace_bytes, stream,
                      "sv_lm_head_greedy launch");
}

static sv_status check_lm_head_pack(int32_t V, int32_t hidden) {
  if (V < 1) return fail(SV_ERR_INVALID_ARG, "V must be >= 1 (got %d)", V);
  if (hidden < 32 || hidden % 32 != 0 || hidden > (1 << 20))
    return fail(SV_ERR_INVALID_ARG, "hidden must be a positive multiple of 32 (got %d)", hidden);
  return SV_OK;
}

sv_status sv_lm_head_pack_bytes(int32_t V, int32_t hidden, size_t* bytes) {
  sv_status st = check_lm_head_pack(V, hidden);
  if (st != SV_OK) return st;
  if (!bytes) return fail(SV_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = sv::lm_head_packed_elems(V, hidden) * 2;
  return ok();
}

sv_status sv_lm_head_pack(int32_t V, int32_t hidden, sv_dtype dtype, const void* weight,
                          void* packed, void* stream) {
  sv_status st = check_lm_head_pack(V, hidden);
  if (st != SV_OK) return st;
  if (!dtype_in(dtype_bits(&dtype), {SV_BF16, SV_F16}))
    return fail(SV_ERR_UNSUPPORTED, "LM head weights must be SV_BF16 or SV_F16");
  if (!weight || !packed) return fail(SV_ERR_INVALID_ARG, "weight and packed are required");
  if (!aligned16(weight) || !aligned16(packed))
    return fail(SV_ERR_INVALID_ARG, "weight and packed must be 16-byte aligned");
  return device_status(sv::launch_lm_head_pack(weight, packed, V, hidden,
                                               static_cast<hipStream_t>(stream)),
                       "sv_lm_head_pack launch");
}

sv_status sv_lm_head_greedy_packed(int32_t B, int32_t K, int32_t V, int32_t hidden,
                                   sv_dtype dtype, const void* hidden_states,
                                   const void* packed_weight, const int32_t* drafts,
                                   int32_t* accept_len, int32_t* out_tokens, int32_t* argmax,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return lm_head_call(B, K, V, hidden, dtype_bits(&dtype), hidden_states, packed_weight, true,
                      drafts, accept_len, out_tokens, argmax, workspace, workspace_bytes, stream,
                      "sv_lm_head_greedy_packed launch");
}

// ---------------------------------------------------------------- sampling
sv_status sv_accept_sample_workspace(int32_t B, int32_t K, int32_t V, size_t* bytes) {
  sv_status st = check_accept_shape(B, K, V, 2);
  if (st != SV_OK) return st;
  if (static_cast<int64_t>(B) * (2 * K - 1) > 65535)
    return fail(SV_ERR_INVALID_ARG, "B * (2K - 1) must be <= 65535");
  if (!bytes) return fail(SV_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = sv::sample_workspace_bytes(B, K, V);
  return ok();
}

sv_status sv_accept_sample(int32_t B, int32_t K, int32_t V, sv_dtype logit_dtype,
                           const void* target_logits, const void* draft_logits,
                           const int32_t* drafts, float temperature, uint64_t seed,
                           uint64_t offset, int32_t* accept_len, int32_t* out_tokens,
                           void* workspace, size_t workspace_bytes, void* stream) {
  sv_status st = check_accept_shape(B, K, V, 2);
  if (st != SV_OK) return st;
  if (static_cast<int64_t>(B) * (2 * K - 1) > 65535)
    return fail(SV_ERR_INVALID_ARG, "B * (2K - 1) must be <= 65535");
  if (!dtype_in(dtype_bits(&logit_dtype), {SV_F32, SV_BF16}))
    return fail(SV_ERR_UNSUPPORTED, "sampling logits must be SV_F32 or SV_BF16");
  if (!(temperature > 0.0f) || !isfinite(temperature))
    return fail(SV_ERR_INVALID_ARG, "temperature must be finite and > 0 (use sv_accept_greedy for 0)");
  if (!target_logits || !draft_logits || !drafts || !accept_len || !out_tokens)
    return fail(SV_ERR_INVALID_ARG, "logits, drafts and outputs are required");
  if (!aligned16(target_logits) || !aligned16(draft_logits))
    return fail(SV_ERR_INVALID_ARG, "target_logits and draft_logits must be 16-byte aligned");
  const int chunk = sv::sample_chunk(V);
  const int nchunk = (V + chunk - 1) / chunk;
  const int race_chunk = sv::sample_race_chunk(V);
  const int race_nchunk = (V + race_chunk - 1) / race_chunk;
  const size_t need = sv::sample_workspace_bytes(B, K, V);
  if (!workspace || workspace_bytes < need)
    return fail(SV_ERR_WORKSPACE, "sampling accept needs %zu workspace bytes", need);
  if (!aligned16(workspace)) return fail(SV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const size_t rows = static_cast<size_t>(B) * (2 * K - 1);
  char* w = static_cast<char*>(workspace);
  sv::SampleParams p;
  p.target = target_logits;
  p.draft = draft_logits;
  p.drafts = drafts;
  p.accept_len = accept_len;
  p.out_tokens = out_tokens;
  p.part_s = reinterpret_cast<double*>(w);
  w += rows * nchunk * sizeof(double);
  p.race_key = reinterpret_cast<double*>(w);
  w += static_cast<size_t>(B) * race_nchunk * 2 * sizeof(double);
  p.part_m = reinterpret_cast<float*>(w);
  w += rows * nchunk * sizeof(float);
  p.race_idx = reinterpret_cast<int32_t*>(w);
  p.B = B;
  p.K = K;
  p.V = V;
  p.chunk = chunk;
  p.nchunk = nchunk;
  p.race_chunk = race_chunk;
  p.race_nchunk = race_nchunk;
  p.inv_t = 1.0 / static_cast<double>(temperature);
  p.wait_limit = sv::wait_limit();
  p.seed = seed;
  p.offset = offset;
  return device_status(sv::launch_sample(p, logit_dtype, static_cast<hipStream_t>(stream)),
                       "sv_accept_sample launch");
}

// ---------------------------------------------------------------- sampling over a tree
sv_status sv_accept_sample_tree_workspace(int32_t B, int32_t K, int32_t V, size_t* bytes) {
  sv_status st = check_accept_shape(B, K, V, 2);
  if (st != SV_OK) return st;
  if (static_cast<int64_t>(B) * (2 * K - 1) > 65535)
    return fail(SV_ERR_INVALID_ARG, "B * (2K - 1) must be <= 65535");
  if (!bytes) return fail(SV_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = sv::sample_tree_workspace_bytes(B, K, V);
  return ok();
}

sv_status sv_accept_sample_tree(int32_t B, int32_t K, int32_t V, sv_dtype logit_dtype,
                                const void* target_logits, const void* draft_logits,
                                const int32_t* parents, const int32_t* tokens, float temperature,
                                uint64_t seed, uint64_t offset, int32_t* accept_len,
                                int32_t* out_tokens, int32_t* accept_path, void* workspace,
                                size_t workspace_bytes, void* stream) {
  sv_status st = check_accept_shape(B, K, V, 2);
  if (st != SV_OK) return st;
  if (static_cast<int64_t>(B) * (2 * K - 1) > 65535)
    return fail(SV_ERR_INVALID_ARG, "B * (2K - 1) must be <= 65535");
  if (!dtype_in(dtype_bits(&logit_dtype), {SV_F32, SV_BF16}))
    return fail(SV_ERR_UNSUPPORTED, "sampling logits must be SV_F32 or SV_BF16");
  if (!(temperature > 0.0f) || !isfinite(temperature))
    return fail(SV_ERR_INVALID_ARG, "temperature must be finite and > 0 (use the greedy calls for 0)");
  if (!target_logits || !draft_logits || !parents || !tokens || !accept_len || !out_tokens ||
      !accept_path)
    return fail(SV_ERR_INVALID_ARG, "logits, parents, tokens and outputs are required");
  if (!aligned16(target_logits) || !aligned16(draft_logits))
    return fail(SV_ERR_INVALID_ARG, "target_logits and draft_logits must be 16-byte aligned");
  for (int i = 1; i < K; ++i)
    if (parents[i - 1] < 0 || parents[i - 1] >= i)
      return fail(SV_ERR_INVALID_ARG, "parents[%d] = %d: the parent of node %d must be in [0, %d)",
                  i - 1, parents[i - 1], i, i);
  const size_t need = sv::sample_tree_workspace_bytes(B, K, V);
  if (!workspace || workspace_bytes < need)
    return fail(SV_ERR_WORKSPACE, "tree sampling needs %zu workspace bytes", need);
  if (!aligned16(workspace)) return fail(SV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  sv::TreeSampleParams p;
  memset(&p, 0, sizeof p);
  p.target = target_logits;
  p.draft = draft_logits;
  p.tokens = tokens;
  p.accept_len = accept_len;
  p.out_tokens = out_tokens;
  p.path = accept_path;
  p.B = B;
  p.K = K;
  p.V = V;
  p.inv_t = 1.0 / static_cast<double>(temperature);
  p.wait_limit = sv::wait_limit();
  p.seed = seed;
  p.offset = offset;
  sv::TreePassPlan plan;
  const int rounds = sv::plan_sample_tree(p, parents, plan);
  if (static_cast<int64_t>(B) * p.nbranch > 65535)
    return fail(SV_ERR_INVALID_ARG, "B times the number of branching nodes must be <= 65535");
  sv::carve_sample_tree_workspace(p, workspace);
  return device_status(sv::launch_sample_tree(p, plan, rounds, logit_dtype,
                                              static_cast<hipStream_t>(stream)),
                       "sv_accept_sample_tree launch");
}

// ---------------------------------------------------------------- compressor
static sv_status check_compress(int32_t B, int32_t C, int32_t N, int32_t D) {
  if (B < 1 || B > 65535) return fail(SV_ERR_INVALID_ARG, "B must be in [1, 65535] (got %d)", B);
  if (C < 1 || C > 64) return fail(SV_ERR_INVALID_ARG, "C must be in [1, 64] (got %d)", C);
  if (N < 1 || N > 1024) return fail(SV_ERR_INVALID_ARG, "N must be in [1, 1024] (got %d)", N);
  if (D < 128 || D % 128 != 0 || D > (1 << 20))
    return fail(SV_ERR_INVALID_ARG, "D must be a positive multiple of 128 (got %d)", D);
  return SV_OK;
}

sv_status sv_latent_compress_workspace(int32_t B, int32_t C, int32_t N, int32_t D, size_t* bytes) {
  sv_status st = check_compress(B, C, N, D);
  if (st != SV_OK) return st;
  if (!bytes) return fail(SV_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = sv::compress_workspace_bytes(B, C, N);
  return ok();
}

sv_status sv_latent_compress(int32_t B, int32_t C, int32_t N, int32_t D, sv_dtype dtype,
                             const void* queries, const void* feats, void* out, float scale,
                             void* workspace, size_t workspace_bytes, void* stream) {
  sv_status st = check_compress(B, C, N, D);
  if (st != SV_OK) return st;
  if (!dtype_in(dtype_bits(&dtype), {SV_F16}))
    return fail(SV_ERR_UNSUPPORTED, "the compressor takes SV_F16 tensors");
  if (!queries || !feats || !out) return fail(SV_ERR_INVALID_ARG, "queries, feats and out are required");
  if (!aligned16(queries) || !aligned16(feats) || !aligned16(out))
    return fail(SV_ERR_INVALID_ARG, "queries, feats and out must be 16-byte aligned");
  if (!(scale >= 0.0f) || !isfinite(scale)) return fail(SV_ERR_INVALID_ARG, "scale must be finite and >= 0");
  const size_t need = sv::compress_workspace_bytes(B, C, N);
  if (!workspace || workspace_bytes < need)
    return fail(SV_ERR_WORKSPACE, "compressor needs %zu workspace bytes", need);
  if (!aligned16(workspace)) return fail(SV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  sv::CompressParams p;
  p.queries = queries;
  p.feats = feats;
  p.out = out;
  p.B = B;
  p.C = C;
  p.N = N;
  p.D = D;
  p.scale = scale > 0.0f ? scale : 1.0f;
  sv::compress_bind_workspace(p, workspace);
  return device_status(sv::launch_compress(p, static_cast<hipStream_t>(stream)),
                       "sv_latent_compress launch");
}

// ---------------------------------------------------------------- KV append
sv_status sv_kv_append(const sv_attn_desc* desc, int32_t n, const void* k_new, const void* v_new,
                       const int32_t* start, const int32_t* page_table, void* k_cache,
                       void* v_cache, void* stream) {
  if (!desc) return fail(SV_ERR_INVALID_ARG, "desc is NULL");
  if (desc->batch < 1 || desc->batch > 65535) return fail(SV_ERR_INVALID_ARG, "batch out of range");
  if (desc->num_kv_heads < 1 || desc->num_kv_heads > 65535)
    return fail(SV_ERR_INVALID_ARG, "num_kv_heads out of range");
  if (desc->head_dim != 64 && desc->head_dim != 128)
    return fail(SV_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!pow2(desc->page_size) || desc->page_size < 16 || desc->page_size > 256)
    return fail(SV_ERR_INVALID_ARG, "page_size must be a power of two in [16, 256]");
  if (desc->max_pages_per_seq < 1 || desc->num_pages < 1)
    return fail(SV_ERR_INVALID_ARG, "max_pages_per_seq and num_pages must be >= 1");
  if (!dtype_in(dtype_bits(&desc->dtype), {SV_F32, SV_BF16, SV_F16}))
    return fail(SV_ERR_UNSUPPORTED, "unknown dtype");
  if (n < 1 || n > 65535) return fail(SV_ERR_INVALID_ARG, "n must be in [1, 65535] (got %d)", n);
  if (!k_new || !v_new || !start || !page_table || !k_cache || !v_cache)
    return fail(SV_ERR_INVALID_ARG, "all arrays are required");
  sv::AppendParams p;
  p.k_new = k_new;
  p.v_new = v_new;
  p.start = start;
  p.page_table = page_table;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.B = desc->batch;
  p.n = n;
  p.Hkv = desc->num_kv_heads;
  p.D = desc->head_dim;
  p.P_log2 = log2i(desc->page_size);
  p.max_pages = desc->max_pages_per_seq;
  p.num_pages = desc->num_pages;
  p.elem_bytes = desc->dtype == SV_F32 ? 4 : 2;
  return device_status(sv::launch_kv_append(p, static_cast<hipStream_t>(stream)),
                       "sv_kv_append launch");
}

// ---------------------------------------------------------------- cycle commit
sv_status sv_commit(int32_t B, int32_t K, const int32_t* accept_len, const int32_t* out_tokens,
                    int32_t* ctx_lens, int32_t* next_anchor, void* stream) {
  if (B < 1 || B > (1 << 24)) return fail(SV_ERR_INVALID_ARG, "B must be in [1, 2^24] (got %d)", B);
  if (K < 1 || K > sv::kMaxBlock) return fail(SV_ERR_INVALID_ARG, "K must be in [1, 64] (got %d)", K);
  if (!accept_len || !out_tokens || !ctx_lens || !next_anchor)
    return fail(SV_ERR_INVALID_ARG, "accept_len, out_tokens, ctx_lens and next_anchor are required");
  sv::CommitParams p;
  p.accept_len = accept_len;
  p.out_tokens = out_tokens;
  p.ctx_lens = ctx_lens;
  p.next_anchor = next_anchor;
  p.B = B;
  p.K = K;
  return device_status(sv::launch_commit(p, static_cast<hipStream_t>(stream)), "sv_commit launch");
}

sv_status sv_commit_tree(const sv_attn_desc* desc, const int32_t* accept_len,
                         const int32_t* out_tokens, const int32_t* accept_path,
                         const int32_t* page_table, void* k_cache, void* v_cache,
                         int32_t* ctx_lens, int32_t* next_anchor, void* stream) {
  if (!desc) return fail(SV_ERR_INVALID_ARG, "desc is NULL");
  const int B = desc->batch, K = desc->block;
  if (B < 1 || B > 65535) return fail(SV_ERR_INVALID_ARG, "batch out of range");
  if (K < 1 || K > sv::kMaxBlock) return fail(SV_ERR_INVALID_ARG, "block must be in [1, 64] (got %d)", K);
  if (desc->num_kv_heads < 1 || desc->num_kv_heads > 65535)
    return fail(SV_ERR_INVALID_ARG, "num_kv_heads out of range");
  if (desc->head_dim != 64 && desc->head_dim != 128)
    return fail(SV_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!pow2(desc->page_size) || desc->page_size < 16 || desc->page_size > 256)
    return fail(SV_ERR_INVALID_ARG, "page_size must be a power of two in [16, 256]");
  if (desc->max_pages_per_seq < 1 || desc->num_pages < 1)
    return fail(SV_ERR_INVALID_ARG, "max_pages_per_seq and num_pages must be >= 1");
  if (!dtype_in(dtype_bits(&desc->dtype), {SV_F32, SV_BF16, SV_F16}))
    return fail(SV_ERR_UNSUPPORTED, "unknown dtype");
  if (!accept_len || !out_tokens || !accept_path || !page_table || !k_cache || !v_cache ||
      !ctx_lens || !next_anchor)
    return fail(SV_ERR_INVALID_ARG, "all arrays are required");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (K > 1) {
    sv::TreeCompactParams t;
    t.accept_len = accept_len;
    t.path = accept_path;
    t.ctx_lens = ctx_lens;
    t.page_table = page_table;
    t.k_cache = k_cache;
    t.v_cache = v_cache;
    t.B = B;
    t.K = K;
    t.Hkv = desc->num_kv_heads;
    t.D = desc->head_dim;
    t.P_log2 = log2i(desc->page_size);
    t.max_pages = desc->max_pages_per_seq;
    t.num_pages = desc->num_pages;
    t.esz = desc->dtype == SV_F32 ? 4 : 2;
    const sv_status st = device_status(sv::launch_tree_compact(t, s), "sv_commit_tree launch");
    if (st != SV_OK) return st;
  }
  sv::CommitParams p;
  p.accept_len = accept_len;
  p.out_tokens = out_tokens;
  p.ctx_lens = ctx_lens;
  p.next_anchor = next_anchor;
  p.B = B;
  p.K = K;
  return device_status(sv::launch_commit(p, s), "sv_commit_tree launch");
}

}  // extern "C"
