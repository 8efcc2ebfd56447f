"""Reference KV append into the paged cache (test infrastructure).

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
