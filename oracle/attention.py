"""Reference block-verification attention in float64 (test infrastructure).

What is computed (VFlash-FM page, "How VFlash-FM works" and the cycle figure:
the unchanged target scores all K block positions in one forward over the full
context plus the block; demo setup: native grouped-query attention, KV caches
preallocated):

For sequence b, block row i in [0, K) and query head h:

* the query head reads KV head g = h // G, G = Hq / Hkv (contiguous head groups);
* visible keys are every context position 0 .. ctx_b - 1, plus block position
  ctx_b + t whenever bit t of mask[i] is set (the default in-block causal mask
  sets bits t <= i, which is what makes row i equal to autoregressive step i);
* s_j = scale * <q, k_j>, scale = 1/sqrt(d) unless given;
* o = sum_j softmax(s)_j v_j and lse = log sum_j exp(s_j).

Cache layout (the library's boundary): K pages [num_pages][Hkv][P][d]
(token-major), V pages [num_pages][Hkv][d][P] (dim-major); token j of sequence
b lives in physical page page_table[b][j // P], slot j % P.
"""
import numpy as np

from .numerics import decode


def _gather(cache_k, cache_v, table_row, n_tokens, P, g):
    """Token-major K [n][d] and V [n][d] of one sequence and KV head."""
    j = np.arange(n_tokens)
    pages = table_row[j // P]
    slots = j % P
    k = cache_k[pages, g, slots, :]            # [n][d]
    v = cache_v[pages, g, :, slots]            # [n][d]
    return k, v


def _visible(mask_rows, ctx, n_tokens):
    """Boolean [K][n]: context always visible, block key t iff bit t of the row mask."""
    K = len(mask_rows)
    vis = np.zeros((K, n_tokens), dtype=bool)
    vis[:, :ctx] = True
    for i in range(K):
        m = int(mask_rows[i])
        for t in range(n_tokens - ctx):
            if (m >> t) & 1:
                vis[i, ctx + t] = True
    return vis


def verify_attention_ref(inp, out_lse: bool = True):
    """Block-causal GQA over a paged cache.

    ``inp`` carries q [B][K][Hq][d], k_cache, v_cache, page_table, ctx_lens,
    mask [K], scale, dtype (see ``workloads.VerifyInputs``).  Returns
    (out float64 [B][K][Hq][d], lse float64 [B][K][Hq]).
    """
    q = decode(inp.q, inp.dtype)
    kc = decode(inp.k_cache, inp.dtype)
    vc = decode(inp.v_cache, inp.dtype)
    B, K, Hq, D = q.shape
    Hkv = kc.shape[1]
    P = kc.shape[2]
    G = Hq // Hkv
    scale = float(inp.scale) if inp.scale else 1.0 / np.sqrt(D)
    out = np.zeros((B, K, Hq, D))
    lse = np.zeros((B, K, Hq))
    for b in range(B):
        ctx = int(inp.ctx_lens[b])
        n = ctx + K
        vis = _visible(inp.mask, ctx, n)
        for h in range(Hq):
            g = h // G
            k, v = _gather(kc, vc, inp.page_table[b], n, P, g)
            s = scale * (q[b, :, h, :] @ k.T)          # [K][n]
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            w = np.exp(s - m)
            l = w.sum(axis=1, keepdims=True)
            out[b, :, h, :] = (w @ v) / l
            lse[b, :, h] = (m + np.log(l))[:, 0]
    return out, lse


def single_query_ref(q_vec, k_rows, v_rows, scale):
    """One query against explicit key/value rows (a plain decode step)."""
    s = scale * (np.asarray(k_rows) @ np.asarray(q_vec))
    m = s.max()
    w = np.exp(s - m)
    return (w @ np.asarray(v_rows)) / w.sum(), m + np.log(w.sum())


def merge_partials_ref(outs, lses):
    """Combine attention results over disjoint key sets.

    With o_s, lse_s the attention of one query over key set s, the attention
    over the union is sum_s exp(lse_s - lse) o_s with lse = log sum_s exp(lse_s).
    """
    lses = np.asarray(lses, dtype=np.float64)
    m = lses.max(axis=0)
    w = np.exp(lses - m)
    tot = w.sum(axis=0)
    out = sum(w[s][..., None] * outs[s] for s in range(len(outs))) / tot[..., None]
    return out, m + np.log(tot)
