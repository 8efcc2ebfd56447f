"""Reference KV append into the paged cache and cycle commit (test infrastructure).

Preallocated KV caches (VFlash-FM page, demo setup): the block's K/V rows are written
into the cache at positions ctx .. ctx+K-1 before the verify forward reads them.  Token
j of sequence b lives in page page_table[b][j // P], slot j % P; K pages are
[num_pages][Hkv][P][d], V pages [num_pages][Hkv][d][P].
"""
import numpy as np


def kv_append_ref(k_cache, v_cache, page_table, start, k_new, v_new):
    """Return copies of the caches with rows [B][n][Hkv][d] written at start[b] + t."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    P = kc.shape[2]
    B, n = k_new.shape[:2]
    for b in range(B):
        for t in range(n):
            j = int(start[b]) + t
            page = int(page_table[b][j // P])
            kc[page, :, j % P, :] = k_new[b, t]
            vc[page, :, :, j % P] = v_new[b, t]
    return kc, vc


def commit_ref(ctx_lens, accept_len, out_tokens):
    """Bookkeeping that closes a verification cycle.

    The accepted drafts plus the target's own token at the first disagreement are the
    committed output, and that last token anchors the next block (VFlash-FM page,
    caption of the cycle figure).  The anchor and the a accepted drafts keep the K/V
    rows written for them before the verify forward, so the context grows by a + 1;
    the rows of rejected drafts are overwritten by the next block's append (the
    preallocated KV cache of the demo setup).

    Returns (new context lengths [B] int32, next anchors [B] int32).
    """
    B = len(ctx_lens)
    new_ctx = np.empty(B, np.int32)
    anchor = np.empty(B, np.int32)
    for b in range(B):
        a = int(accept_len[b])
        new_ctx[b] = int(ctx_lens[b]) + a + 1
        anchor[b] = int(out_tokens[b][a])
    return new_ctx, anchor
