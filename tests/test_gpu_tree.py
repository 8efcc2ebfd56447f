"""GPU parity of draft-tree verification against the float64 oracle (needs an MI355X):
tree-masked attention (up to 2 row groups of 256 rows per KV head, 4 of 128 for fp32), the greedy tree walk,
the tree commit, and chained device-resident tree cycles."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import check_attention, i32, say, to_dev, upload_verify

pytestmark = pytest.mark.gpu


def _levels(n, rng):
    """Split n draft nodes into 2..6 non-empty levels."""
    depth = int(rng.integers(2, 7))
    depth = min(depth, n)
    cuts = np.sort(rng.choice(np.arange(1, n), size=depth - 1, replace=False)) if depth > 1 else []
    edges = [0] + list(cuts) + [n]
    return tuple(int(edges[i + 1] - edges[i]) for i in range(depth))


def _verify(sv, inp, split_keys=0):
    d = upload_verify(inp)
    out, lse = sv.verify_attention(d["q"], d["k_cache"], d["v_cache"], d["page_table"],
                                   d["ctx_lens"], max_ctx=int(inp.ctx_lens.max()),
                                   block_mask=inp.mask, split_keys=split_keys,
                                   sum_ctx_hint=int(inp.ctx_lens.sum()))
    torch.cuda.synchronize()
    return out, lse


def test_tree60_layer_full_size(gpu_lib):
    """The 7B layer verifying Tree-60: 61 rows x 7 query heads = 427 rows per KV head."""
    inp = W.make_workload_verify("qwen7b_tree60")
    say(f"[tree attention] qwen7b_tree60 ctx={list(inp.ctx_lens)} K={inp.K}")
    out, lse = _verify(gpu_lib, inp)
    ref_out, ref_lse = oracle.verify_attention_ref(inp)
    worst, ratio = check_attention(out, lse, ref_out, ref_lse, inp.dtype, "qwen7b_tree60")
    say(f"  max|d|={worst:.2e} slice-rel={ratio:.2e}")


TREE_CASES = [
    # dtype, D, P, Hq, Hkv, K, ctx, split_keys
    ("bf16", 128, 16, 28, 4, 61, [1000], 0),        # 427 rows: 2 row groups of 256
    ("bf16", 128, 16, 28, 4, 40, [777, 31], 64),    # 280 rows: 2 row groups, many splits
    ("bf16", 64, 16, 32, 2, 20, [400, 90], 0),      # 320 rows at d 64, two sequences
    ("f32", 128, 16, 28, 4, 40, [300], 0),          # 280 rows, fp32: 3 row groups of 128
    ("f16", 128, 32, 16, 2, 60, [300], 0),          # 480 rows
    ("f32", 64, 16, 16, 2, 64, [130, 5], 32),       # 512 rows (the limit), fp32
    ("bf16", 64, 16, 8, 8, 13, [0], 0),             # empty context, G = 1
]


@pytest.mark.parametrize("case", TREE_CASES, ids=[f"t{i}" for i in range(len(TREE_CASES))])
def test_tree_masks(gpu_lib, case):
    dtype, D, P, Hq, Hkv, K, ctx, split = case
    rng = np.random.default_rng(300 + TREE_CASES.index(case))
    parents = W.make_tree_topology(rng, _levels(K - 1, rng))
    inp = W.make_verify(rng, B=len(ctx), K=K, Hq=Hq, Hkv=Hkv, D=D, ctx_lens=ctx, P=P,
                        dtype=dtype, shuffle=True, mask=W.tree_mask(parents))
    say(f"[tree attention] case={case}")
    out, lse = _verify(gpu_lib, inp, split)
    ref_out, ref_lse = oracle.verify_attention_ref(inp)
    check_attention(out, lse, ref_out, ref_lse, dtype, str(case))


def _check_tree_accept(gpu, ti, dtype):
    acc, toks, path, am = gpu.accept_greedy_tree(to_dev(ti.logits, dtype), i32(ti.parents),
                                                 i32(ti.tokens))
    torch.cuda.synchronize()
    r_acc, r_toks, r_path, r_am = oracle.accept_greedy_tree_ref(ti.logits, ti.parents,
                                                                ti.tokens, dtype)
    np.testing.assert_array_equal(am.cpu().numpy(), r_am)
    np.testing.assert_array_equal(acc.cpu().numpy(), r_acc)
    np.testing.assert_array_equal(toks.cpu().numpy(), r_toks)
    np.testing.assert_array_equal(path.cpu().numpy(), r_path)
    return r_acc


def test_tree60_accept_full_size(gpu_lib):
    ti = W.make_workload_tree("qwen7b_tree60")
    say(f"[tree accept] qwen7b_tree60 K={ti.K} V={ti.V}")
    _check_tree_accept(gpu_lib, ti, ti.dtype)


@pytest.mark.parametrize("seed,B,K,V,dtype", [
    (0, 16, 61, 1000, "bf16"), (1, 8, 64, 3000, "f32"), (2, 5, 2, 50, "bf16"),
    (3, 32, 31, 152064, "bf16"), (4, 3, 20, 100003, "f32"),
])
def test_tree_accept(gpu_lib, seed, B, K, V, dtype):
    rng = np.random.default_rng(400 + seed)
    parents = W.make_tree_topology(rng, _levels(K - 1, rng)) if K > 2 else np.zeros(1, np.int32)
    ti = W.make_tree_greedy(rng, B=B, V=V, parents=parents, dtype=dtype)
    say(f"[tree accept] seed={seed} B={B} K={K} V={V} {dtype}")
    r_acc = _check_tree_accept(gpu_lib, ti, dtype)
    np.testing.assert_array_equal(r_acc, ti.planted_len)


def test_tree_accept_edge_cases(gpu_lib):
    rng = np.random.default_rng(450)
    V = 40
    # a chain given as a tree: the chain rule's results
    g = W.make_greedy(rng, B=6, K=16, V=V, dtype="f32")
    parents = np.tile(W.chain_topology(15), (6, 1))
    acc, toks, path, am = gpu_lib.accept_greedy_tree(to_dev(g.logits, "f32"), i32(parents),
                                                     i32(g.drafts))
    c_acc, c_toks, c_am = gpu_lib.accept_greedy(to_dev(g.logits, "f32"), i32(g.drafts))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), c_acc.cpu().numpy())
    np.testing.assert_array_equal(toks.cpu().numpy(), c_toks.cpu().numpy())
    # duplicate sibling tokens (the lower-numbered child wins); and parents that are not
    # a tree: node 2 names itself, node 3 names the later node 5 and holds node 5's greedy
    # token, yet the walk never steps back to it (expected values worked out by hand)
    x = rng.normal(0, 1, size=(2, 6, V)).astype(np.float32)
    for i, t in enumerate([3, 4, 1, 1, 0, 1]):
        x[:, i, t] = 10.0
    par = np.array([[0, 0, 1, 1, 4], [0, 2, 5, 1, 4]], np.int32)
    tok = np.array([[3, 3, 2, 4, 0], [3, 3, 1, 4, 0]], np.int32)
    acc, toks, path, am = gpu_lib.accept_greedy_tree(to_dev(x, "f32"), i32(par), i32(tok))
    torch.cuda.synchronize()
    assert acc.cpu().tolist() == [3, 3]
    assert path.cpu().tolist() == [[0, 1, 4, 5, -1, -1]] * 2
    assert toks.cpu().tolist() == [[3, 4, 0, 1, -1, -1]] * 2
    # the anchor alone (K = 1)
    x1 = rng.normal(0, 1, size=(3, 1, V)).astype(np.float32)
    acc, toks, path, _ = gpu_lib.accept_greedy_tree(to_dev(x1, "f32"),
                                                    torch.zeros(3, 0, dtype=torch.int32, device="cuda"),
                                                    torch.zeros(3, 0, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert acc.cpu().tolist() == [0, 0, 0] and path.cpu().tolist() == [[0]] * 3
    assert toks.cpu().numpy()[:, 0].tolist() == x1[:, 0].argmax(axis=1).tolist()


@pytest.mark.parametrize("dtype,D,P", [("bf16", 128, 16), ("f32", 64, 32)])
def test_tree_commit(gpu_lib, dtype, D, P):
    rng = np.random.default_rng(500 + D)
    parents = W.make_tree_topology(rng, (5, 8, 6, 4, 3, 2))
    K = len(parents) + 1
    B, Hkv = 6, 4
    ctx = np.array([0, 17, 250, 33, 1000, 5], np.int32)
    inp = W.make_verify(rng, B=B, K=K, Hq=Hkv, Hkv=Hkv, D=D, ctx_lens=ctx, P=P, dtype=dtype,
                        shuffle=True)
    ti = W.make_tree_greedy(rng, B=B, V=300, parents=parents, dtype="bf16")
    say(f"[tree commit] {dtype} D={D} P={P} planted={ti.planted_len.tolist()}")
    acc, toks, path, _ = gpu_lib.accept_greedy_tree(to_dev(ti.logits, "bf16"), i32(ti.parents),
                                                    i32(ti.tokens))
    kc, vc = to_dev(inp.k_cache, dtype), to_dev(inp.v_cache, dtype)
    ctx_dev = i32(ctx)
    anchor = gpu_lib.commit_tree(acc, toks, path, i32(inp.page_table), kc, vc, ctx_dev)
    torch.cuda.synchronize()
    r_acc, r_toks, r_path, _ = oracle.accept_greedy_tree_ref(ti.logits, ti.parents, ti.tokens,
                                                             "bf16")
    rk, rv, r_ctx, r_anchor = oracle.tree_commit_ref(inp.k_cache, inp.v_cache, inp.page_table,
                                                     ctx, r_acc, r_toks, r_path)
    np.testing.assert_array_equal(ctx_dev.cpu().numpy(), r_ctx)
    np.testing.assert_array_equal(anchor.cpu().numpy(), r_anchor)
    view = (lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)) if dtype == "bf16" \
        else (lambda t: t.cpu().numpy())
    np.testing.assert_array_equal(view(kc), rk)
    np.testing.assert_array_equal(view(vc), rv)


def test_chained_tree_cycles(gpu_lib):
    """Append the tree's node rows at the device context, verify with the tree mask,
    walk, commit -- three cycles, state on the device, against the oracle's chain."""
    rng = np.random.default_rng(2025)
    B, Hq, Hkv, D, P, V = 2, 28, 4, 128, 16, 4000
    parents = W.make_tree_topology(rng, W.TREE60_LEVELS)
    K = len(parents) + 1
    mask = W.tree_mask(parents)
    cycles = 3
    ctx0 = np.array([500, 64], dtype=np.int32)
    cap = int(ctx0.max()) + (cycles + 1) * K
    inp = W.make_verify(rng, B=B, K=K, Hq=Hq, Hkv=Hkv, D=D, ctx_lens=[cap - K] * B, P=P,
                        dtype="bf16", shuffle=True)
    kc_ref, vc_ref = inp.k_cache.copy(), inp.v_cache.copy()
    kc, vc = to_dev(kc_ref, "bf16"), to_dev(vc_ref, "bf16")
    pt = i32(inp.page_table)
    ctx_dev = i32(ctx0)
    ctx_ref = ctx0.copy()
    for c in range(cycles):
        say(f"[tree cycle] {c}: ctx {ctx_ref.tolist()}")
        k_new = W.bf16_bits(rng.standard_normal((B, K, Hkv, D), dtype=np.float32))
        v_new = W.bf16_bits(rng.standard_normal((B, K, Hkv, D), dtype=np.float32))
        q = W.bf16_bits(rng.standard_normal((B, K, Hq, D), dtype=np.float32))
        gpu_lib.kv_append(to_dev(k_new, "bf16"), to_dev(v_new, "bf16"), ctx_dev, pt, kc, vc)
        out, lse = gpu_lib.verify_attention(to_dev(q, "bf16"), kc, vc, pt, ctx_dev,
                                            max_ctx=cap - K, block_mask=mask)
        kc_ref, vc_ref = oracle.kv_append_ref(kc_ref, vc_ref, inp.page_table, ctx_ref, k_new, v_new)
        step = W.VerifyInputs(B, K, Hq, Hkv, D, P, "bf16", q, kc_ref, vc_ref, inp.page_table,
                              ctx_ref.copy(), mask)
        ref_out, ref_lse = oracle.verify_attention_ref(step)
        torch.cuda.synchronize()
        check_attention(out, lse, ref_out, ref_lse, "bf16", f"tree cycle {c}")
        ti = W.make_tree_greedy(rng, B=B, V=V, parents=parents, dtype="bf16")
        acc, toks, path, _ = gpu_lib.accept_greedy_tree(to_dev(ti.logits, "bf16"),
                                                        i32(ti.parents), i32(ti.tokens))
        anchor = gpu_lib.commit_tree(acc, toks, path, pt, kc, vc, ctx_dev)
        r_acc, r_toks, r_path, _ = oracle.accept_greedy_tree_ref(ti.logits, ti.parents,
                                                                 ti.tokens, "bf16")
        kc_ref, vc_ref, ctx_ref, r_anchor = oracle.tree_commit_ref(
            kc_ref, vc_ref, inp.page_table, ctx_ref, r_acc, r_toks, r_path)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc.cpu().numpy(), r_acc)
        np.testing.assert_array_equal(anchor.cpu().numpy(), r_anchor)
        np.testing.assert_array_equal(ctx_dev.cpu().numpy(), ctx_ref)
    np.testing.assert_array_equal(kc.view(torch.int16).cpu().numpy().view(np.uint16), kc_ref)
    np.testing.assert_array_equal(vc.view(torch.int16).cpu().numpy().view(np.uint16), vc_ref)
