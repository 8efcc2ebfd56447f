"""Pins of the attention oracle against things other than itself (CPU only)."""
import copy

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _small(seed, B=2, K=4, Hq=4, Hkv=2, D=16, ctx=(13, 29), P=4, dtype="f32", shuffle=True,
           mask=None):
    rng = np.random.default_rng(seed)
    return W.make_verify(rng, B=B, K=K, Hq=Hq, Hkv=Hkv, D=D, ctx_lens=list(ctx)[:B], P=P,
                         dtype=dtype, shuffle=shuffle, mask=mask)


def _token_major(inp, b, g):
    """Token-major K/V of one sequence, read through the page table."""
    kc = oracle.decode(inp.k_cache, inp.dtype)
    vc = oracle.decode(inp.v_cache, inp.dtype)
    n = int(inp.ctx_lens[b]) + inp.K
    ks = np.stack([kc[inp.page_table[b][j // inp.P], g, j % inp.P, :] for j in range(n)])
    vs = np.stack([vc[inp.page_table[b][j // inp.P], g, :, j % inp.P] for j in range(n)])
    return ks, vs


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("mask_kind", ["causal", "ones", "random"])
def test_vs_torch_sdpa_gqa(dtype, mask_kind):
    """Library route: torch SDPA in float64 with enable_gqa (head h reads KV head h // G)."""
    K = 5
    rng = np.random.default_rng(7)
    if mask_kind == "causal":
        mask = W.causal_mask(K)
    elif mask_kind == "ones":
        mask = W.all_ones_mask(K)
    else:
        mask = np.array([(int(rng.integers(0, 1 << K)) | (1 << i)) for i in range(K)],
                        dtype=np.uint64)
    inp = _small(11, K=K, Hq=6, Hkv=2, dtype=dtype, mask=mask)
    out, lse = oracle.verify_attention_ref(inp)
    q = oracle.decode(inp.q, dtype)
    for b in range(inp.B):
        ctx = int(inp.ctx_lens[b])
        n = ctx + K
        ks, vs = zip(*[_token_major(inp, b, g) for g in range(inp.Hkv)])
        kt = torch.tensor(np.stack(ks))            # [Hkv][n][D]
        vt = torch.tensor(np.stack(vs))
        qt = torch.tensor(q[b].transpose(1, 0, 2))  # [Hq][K][D]
        allowed = torch.zeros(K, n, dtype=torch.bool)
        allowed[:, :ctx] = True
        for i in range(K):
            for t in range(K):
                if (int(mask[i]) >> t) & 1:
                    allowed[i, ctx + t] = True
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt[None], kt[None], vt[None], attn_mask=allowed, enable_gqa=True)[0]
        np.testing.assert_allclose(out[b].transpose(1, 0, 2), ref.numpy(), rtol=1e-12,
                                   atol=1e-12)
        # lse through torch.logsumexp of the masked score matrix
        rep = kt.repeat_interleave(inp.Hq // inp.Hkv, dim=0)
        s = (qt @ rep.transpose(1, 2)) / np.sqrt(inp.D)
        s = s.masked_fill(~allowed, float("-inf"))
        np.testing.assert_allclose(lse[b].T, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12,
                                   atol=1e-12)


def test_split_merge_invariance():
    """Attention over a key set equals the LSE-weighted merge over any partition of it."""
    inp = _small(3, B=1, K=3, Hq=2, Hkv=1, D=8, ctx=(40,), P=4, shuffle=False)
    out, lse = oracle.verify_attention_ref(inp)
    scale = 1 / np.sqrt(inp.D)
    q = oracle.decode(inp.q, inp.dtype)
    ks, vs = _token_major(inp, 0, 0)
    ctx = int(inp.ctx_lens[0])
    rng = np.random.default_rng(5)
    for i in range(inp.K):
        vis = list(range(ctx + i + 1))
        cuts = np.sort(rng.choice(np.arange(1, len(vis)), size=6, replace=False))
        parts = np.split(np.array(vis), cuts)
        for h in range(inp.Hq):
            os_, ls_ = zip(*[oracle.single_query_ref(q[0, i, h], ks[p], vs[p], scale)
                             for p in parts])
            mo, ml = oracle.merge_partials_ref(list(os_), list(ls_))
            np.testing.assert_allclose(mo, out[0, i, h], rtol=1e-12, atol=1e-13)
            assert abs(ml - lse[0, i, h]) < 1e-12


def test_block_row_equals_decode_step():
    """Row i of a causal block equals a single-query step over keys [0, ctx + i]."""
    inp = _small(9, B=2, K=6, Hq=4, Hkv=2, D=16, ctx=(21, 8), P=4)
    out, lse = oracle.verify_attention_ref(inp)
    for b in range(inp.B):
        ctx = int(inp.ctx_lens[b])
        for i in range(inp.K):
            one = copy.copy(inp)
            one.B = 1
            one.K = 1
            one.q = inp.q[b:b + 1, i:i + 1]
            one.page_table = inp.page_table[b:b + 1]
            one.ctx_lens = np.array([ctx + i], dtype=np.int32)
            one.mask = W.causal_mask(1)
            o1, l1 = oracle.verify_attention_ref(one)
            np.testing.assert_allclose(o1[0, 0], out[b, i], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(l1[0, 0], lse[b, i], rtol=1e-12, atol=1e-13)


def test_page_permutation_invariance():
    """Moving pages to other physical slots (and fixing the table) changes nothing."""
    inp = _small(4, shuffle=False)
    out, lse = oracle.verify_attention_ref(inp)
    perm = np.random.default_rng(1).permutation(inp.num_pages)
    moved = copy.copy(inp)
    moved.k_cache = np.empty_like(inp.k_cache)
    moved.v_cache = np.empty_like(inp.v_cache)
    moved.k_cache[perm] = inp.k_cache
    moved.v_cache[perm] = inp.v_cache
    moved.page_table = np.where(inp.page_table >= 0, perm[inp.page_table], -1).astype(np.int32)
    o2, l2 = oracle.verify_attention_ref(moved)
    np.testing.assert_array_equal(out, o2)
    np.testing.assert_array_equal(lse, l2)


def test_closed_forms():
    # (1) identical keys: uniform softmax -> mean of the visible values; lse = s + log n
    inp = _small(2, B=1, K=3, Hq=2, Hkv=1, D=8, ctx=(10,), P=4, shuffle=False)
    inp.k_cache[:] = inp.k_cache[0, 0, 0]
    out, lse = oracle.verify_attention_ref(inp)
    ks, vs = _token_major(inp, 0, 0)
    q = oracle.decode(inp.q, "f32")
    for i in range(3):
        n = 10 + i + 1
        for h in range(2):
            np.testing.assert_allclose(out[0, i, h], vs[:n].mean(axis=0), rtol=1e-12, atol=1e-13)
            s = q[0, i, h] @ ks[0] / np.sqrt(8)
            assert abs(lse[0, i, h] - (s + np.log(n))) < 1e-12
    # (2) empty context, one block row: the only visible key's value
    inp = _small(3, B=1, K=1, Hq=2, Hkv=1, D=8, ctx=(0,), P=4, shuffle=False)
    out, _ = oracle.verify_attention_ref(inp)
    ks, vs = _token_major(inp, 0, 0)
    np.testing.assert_allclose(out[0, 0, 0], vs[0], rtol=0, atol=1e-15)
    # (3) a query aligned with one key, scaled up: the output tends to that key's value
    inp = _small(6, B=1, K=1, Hq=1, Hkv=1, D=32, ctx=(20,), P=4, shuffle=False)
    ks, vs = _token_major(inp, 0, 0)
    inp.q = (ks[7] * 50.0).astype(np.float32)[None, None, None, :]
    out, _ = oracle.verify_attention_ref(inp)
    np.testing.assert_allclose(out[0, 0, 0], vs[7], atol=1e-6)


def test_mask_rows_respected():
    """A block key hidden from a row cannot move that row's output."""
    K = 4
    mask = np.array([0b0001, 0b0011, 0b0101, 0b1001], dtype=np.uint64)
    inp = _small(8, B=1, K=K, Hq=2, Hkv=1, D=8, ctx=(12,), P=4, shuffle=False, mask=mask)
    out, _ = oracle.verify_attention_ref(inp)
    pert = copy.deepcopy(inp)
    # overwrite block keys 1 and 2 (positions ctx+1, ctx+2): only rows that see them may change
    for t in (1, 2):
        j = 12 + t
        pert.k_cache[pert.page_table[0][j // 4], 0, j % 4, :] += 3.0
        pert.v_cache[pert.page_table[0][j // 4], 0, :, j % 4] -= 2.0
    o2, _ = oracle.verify_attention_ref(pert)
    for i in range(K):
        sees = any((int(mask[i]) >> t) & 1 for t in (1, 2))
        changed = not np.allclose(out[0, i], o2[0, i], atol=0, rtol=0)
        assert changed == sees, (i, sees, changed)


def test_kv_append_round_trip():
    """Rows appended at positions p are what the attention oracle gathers at p: a block
    appended after the context gives the same attention as a cache built with it."""
    inp = _small(21, B=2, K=3, Hq=2, Hkv=2, D=8, ctx=(10, 5), P=4)
    rng = np.random.default_rng(3)
    new_k = rng.standard_normal((2, 3, 2, 8)).astype(np.float32)
    new_v = rng.standard_normal((2, 3, 2, 8)).astype(np.float32)
    kc, vc = oracle.kv_append_ref(inp.k_cache, inp.v_cache, inp.page_table, inp.ctx_lens,
                                  new_k, new_v)
    moved = copy.copy(inp)
    moved.k_cache, moved.v_cache = kc, vc
    for b in range(2):
        for g in range(2):
            ks, vs = _token_major(moved, b, g)
            ctx = int(inp.ctx_lens[b])
            np.testing.assert_array_equal(ks[ctx:ctx + 3], new_k[b, :, g])
            np.testing.assert_array_equal(vs[ctx:ctx + 3], new_v[b, :, g])
            k0, v0 = _token_major(inp, b, g)
            np.testing.assert_array_equal(ks[:ctx], k0[:ctx])     # context untouched
            np.testing.assert_array_equal(vs[:ctx], v0[:ctx])
