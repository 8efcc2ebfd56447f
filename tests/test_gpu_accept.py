"""GPU parity of sv_accept_greedy / sv_accept_sample against the oracle: bit-exact."""
import json
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import i32, say, to_dev

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))

pytestmark = pytest.mark.gpu


def greedy_gpu(sv, logits, drafts, dtype):
    acc, toks, am = sv.accept_greedy(to_dev(logits, dtype), i32(drafts))
    torch.cuda.synchronize()
    return acc.cpu().numpy(), toks.cpu().numpy(), am.cpu().numpy()


def assert_greedy(sv, logits, drafts, dtype, where):
    acc, toks, am = greedy_gpu(sv, logits, drafts, dtype)
    r_acc, r_toks, r_am = oracle.accept_greedy_ref(logits, drafts, dtype)
    np.testing.assert_array_equal(am, r_am, err_msg=f"{where}: argmax")
    np.testing.assert_array_equal(acc, r_acc, err_msg=f"{where}: accept_len")
    np.testing.assert_array_equal(toks, r_toks, err_msg=f"{where}: out_tokens")
    return acc


@pytest.mark.parametrize("name", ["tiny_fp32", "qwen7b_25k", "batched_paged"])
def test_greedy_named_workloads(gpu_lib, name):
    for cycle in range(3):
        g = W.make_workload_greedy(name, cycle)
        say(f"[greedy] workload={name} cycle={cycle} B={g.B} K={g.K} V={g.V}")
        acc = assert_greedy(gpu_lib, g.logits, g.drafts, g.dtype, f"{name}/{cycle}")
        np.testing.assert_array_equal(acc, g.planted_len)


@pytest.mark.parametrize("B,K,V,dtype", [
    (4, 16, 1001, "bf16"),      # V not a multiple of 8: scalar path
    (3, 8, 999, "f32"),
    (2, 4, 1, "bf16"),          # one-token vocabulary
    (5, 1, 5000, "bf16"),       # K = 1: no drafts, the target's token only
    (64, 16, 20000, "bf16"),    # many sequences
    (2, 64, 9000, "f32"),       # K = 64
    (2, 8, 150000, "f32"),      # several load rounds per vocabulary chunk
    (1, 4, 300000, "bf16"),
])
def test_greedy_shapes(gpu_lib, B, K, V, dtype):
    rng = np.random.default_rng(B * 1000 + K)
    g = W.make_greedy(rng, B=B, K=K, V=V, dtype=dtype)
    say(f"[greedy] B={B} K={K} V={V} {dtype}")
    assert_greedy(gpu_lib, g.logits, g.drafts, dtype, f"{B},{K},{V}")


def test_greedy_ties_across_chunks_and_signed_zero(gpu_lib):
    """Equal maxima in different vocabulary chunks (different workgroups) and +-0.0."""
    K, V = 4, 40000
    x = np.full((1, K, V), -1.0, dtype=np.float32)
    x[0, 0, [30000, 9000, 17]] = 7.0           # lowest index 17, far apart
    x[0, 1, [39999, 8192]] = 7.0               # chunk-boundary index 8192 wins
    x[0, 2, :] = -2.0
    x[0, 2, [5, 20000]] = 0.0
    x[0, 2, 3] = -0.0                          # -0.0 equals +0.0: index 3 wins
    x[0, 3, V - 1] = 3.0
    drafts = np.array([[17, 8192, 3]], dtype=np.int32)
    say("[greedy] ties / signed zero")
    for dtype in ("f32", "bf16"):
        logits = x if dtype == "f32" else W.bf16_bits(x)
        acc, toks, am = greedy_gpu(gpu_lib, logits, drafts, dtype)
        assert list(am[0]) == [17, 8192, 3, V - 1]
        assert acc[0] == 3 and list(toks[0]) == [17, 8192, 3, V - 1]
        assert_greedy(gpu_lib, logits, drafts, dtype, f"ties/{dtype}")


def test_greedy_workspace_reuse(gpu_lib):
    """Back-to-back calls of different shapes share the cached workspace, which carries
    no state from one call to the next."""
    for i, (B, K, V) in enumerate([(2, 16, 3000), (8, 4, 500), (2, 16, 3000), (1, 64, 700)]):
        g = W.make_greedy(np.random.default_rng(50 + i), B=B, K=K, V=V, dtype="bf16")
        say(f"[greedy] reuse {i}")
        for _ in range(3):
            assert_greedy(gpu_lib, g.logits, g.drafts, "bf16", f"reuse{i}")


def test_greedy_workspace_garbage_and_graph_replays(gpu_lib):
    """The workspace needs no initial contents: calls on a workspace filled with 0xFF bytes,
    with random bytes and with zeros match the oracle.  One call captured in a HIP graph
    and replayed five times, with new logits copied in eagerly between replays, matches
    the oracle on every replay."""
    import ctypes
    B, K, V = 3, 16, 50000
    n = ctypes.c_size_t()
    assert gpu_lib.load().sv_accept_greedy_workspace(B, K, V, ctypes.byref(n)) == 0
    gs = [W.make_greedy(np.random.default_rng(900 + i), B=B, K=K, V=V, dtype="bf16")
          for i in range(6)]
    gen = torch.Generator(device="cpu").manual_seed(5)
    fills = [torch.full((n.value,), 0xFF, dtype=torch.uint8),
             torch.randint(0, 256, (n.value,), dtype=torch.uint8, generator=gen),
             torch.zeros(n.value, dtype=torch.uint8)]
    for i, fill in enumerate(fills):
        say(f"[greedy] workspace fill {i}")
        ws = fill.cuda()
        acc, toks, am = gpu_lib.accept_greedy(to_dev(gs[i].logits, "bf16"), i32(gs[i].drafts),
                                              workspace=ws)
        torch.cuda.synchronize()
        r_acc, r_toks, r_am = oracle.accept_greedy_ref(gs[i].logits, gs[i].drafts, "bf16")
        np.testing.assert_array_equal(am.cpu().numpy(), r_am)
        np.testing.assert_array_equal(acc.cpu().numpy(), r_acc)
        np.testing.assert_array_equal(toks.cpu().numpy(), r_toks)
    say("[greedy] graph replays")
    logits = to_dev(gs[0].logits, "bf16")
    drafts = i32(gs[0].drafts)
    ws = torch.full((n.value,), 0xA5, dtype=torch.uint8, device="cuda")
    outs = (torch.empty(B, dtype=torch.int32, device="cuda"),
            torch.empty(B, K, dtype=torch.int32, device="cuda"),
            torch.empty(B, K, dtype=torch.int32, device="cuda"))
    st = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        gpu_lib.accept_greedy(logits, drafts, out=outs, workspace=ws, stream=st)
    for r in range(5):
        g = gs[1 + r]
        logits.copy_(to_dev(g.logits, "bf16"))
        drafts.copy_(i32(g.drafts))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        r_acc, r_toks, r_am = oracle.accept_greedy_ref(g.logits, g.drafts, "bf16")
        np.testing.assert_array_equal(outs[2].cpu().numpy(), r_am, err_msg=f"replay {r}")
        np.testing.assert_array_equal(outs[0].cpu().numpy(), r_acc, err_msg=f"replay {r}")
        np.testing.assert_array_equal(outs[1].cpu().numpy(), r_toks, err_msg=f"replay {r}")


# ------------------------------------------------------------------------- sampling
def sample_gpu(sv, s):
    acc, toks = sv.accept_sample(to_dev(s.target_logits, s.dtype), to_dev(s.draft_logits, s.dtype),
                                 i32(s.drafts), s.temperature, s.seed, s.offset)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), toks.cpu().numpy()


def assert_sample(sv, s, where):
    acc, toks = sample_gpu(sv, s)
    r_acc, r_toks, diag = oracle.accept_sample_ref(s.target_logits, s.draft_logits, s.drafts,
                                                   s.dtype, s.temperature, s.seed, s.offset,
                                                   return_diag=True)
    margins = [m for m, _ in diag]
    gaps = [gp for _, gp in diag]
    msg = (f"{where}: accept {acc} vs {r_acc}; smallest |u - ratio| {min(margins):.3e}, "
           f"smallest race gap {min(gaps):.3e}")
    np.testing.assert_array_equal(acc, r_acc, err_msg=msg)
    np.testing.assert_array_equal(toks, r_toks, err_msg=msg)
    return acc, min(margins), min(gaps)


def test_sample_72b_workload(gpu_lib):
    """Full vocabulary, K = 32, temperature 1: several cycles (Philox offsets)."""
    accs = []
    for cycle in range(6):
        s = W.make_workload_sample("qwen72b_sampling", cycle)
        say(f"[sample] qwen72b cycle={cycle} V={s.V} K={s.K}")
        acc, m, gp = assert_sample(gpu_lib, s, f"72b/{cycle}")
        accs.append(int(acc[0]))
        say(f"  accept_len={acc[0]} margin={m:.2e} gap={gp:.2e}")


@pytest.mark.parametrize("B,K,V,dtype,T", [
    (16, 8, 1000, "bf16", 1.0),
    (16, 4, 5000, "f32", 0.7),
    (8, 16, 3001, "bf16", 1.5),
    (32, 2, 257, "f32", 1.0),
    (4, 32, 20000, "bf16", 1.0),
])
def test_sample_many_cycles(gpu_lib, B, K, V, dtype, T):
    rng = np.random.default_rng(B + K + V)
    total = 0
    for off in range(12):
        s = W.make_sample(rng, B=B, K=K, V=V, dtype=dtype, temperature=T, seed=0x5EED + B,
                          offset=off)
        say(f"[sample] B={B} K={K} V={V} {dtype} T={T} offset={off}")
        acc, _, _ = assert_sample(gpu_lib, s, f"{B},{K},{V},{T},{off}")
        total += int(acc.sum())
    assert total > 0


def test_sample_q_equals_p(gpu_lib):
    rng = np.random.default_rng(9)
    s = W.make_sample(rng, B=8, K=6, V=4000, dtype="bf16", noise=0.0, seed=3, offset=1)
    say("[sample] q == p")
    acc, toks = sample_gpu(gpu_lib, s)
    assert (acc == 5).all()
    np.testing.assert_array_equal(toks[:, :5], s.drafts)
    assert_sample(gpu_lib, s, "q==p")


def test_sample_deterministic_and_offset_sensitive(gpu_lib):
    rng = np.random.default_rng(10)
    s = W.make_sample(rng, B=16, K=8, V=2000, dtype="bf16", seed=77, offset=5)
    say("[sample] determinism")
    a1 = sample_gpu(gpu_lib, s)
    a2 = sample_gpu(gpu_lib, s)
    np.testing.assert_array_equal(a1[0], a2[0])
    np.testing.assert_array_equal(a1[1], a2[1])
    s.offset = 6
    a3 = sample_gpu(gpu_lib, s)
    assert not np.array_equal(a1[1], a3[1])


def test_sample_workspace_garbage_and_graph_replays(gpu_lib):
    """The last race workgroup of each sequence waits on its sequence's winner slots, which
    the first launch of every call empties: calls on workspaces filled with 0xFF bytes,
    with random bytes and with the empty-slot pattern itself match the oracle, and one
    call captured in a HIP graph and replayed four times, with new logits copied in
    eagerly between replays, matches the oracle on every replay."""
    import ctypes
    B, K, V = 4, 8, 20000
    n = ctypes.c_size_t()
    assert gpu_lib.load().sv_accept_sample_workspace(B, K, V, ctypes.byref(n)) == 0
    ss = [W.make_sample(np.random.default_rng(700 + i), B=B, K=K, V=V, dtype="bf16",
                        seed=11, offset=i) for i in range(7)]
    gen = torch.Generator(device="cpu").manual_seed(6)
    empty = np.frombuffer(np.array([0x7FF5A5A5A5A5A5A5], np.uint64).tobytes(), np.uint8)
    fills = [torch.full((n.value,), 0xFF, dtype=torch.uint8),
             torch.randint(0, 256, (n.value,), dtype=torch.uint8, generator=gen),
             torch.from_numpy(np.resize(empty, n.value).copy())]
    for i, fill in enumerate(fills):
        say(f"[sample] workspace fill {i}")
        s = ss[i]
        acc, toks = gpu_lib.accept_sample(to_dev(s.target_logits, "bf16"),
                                          to_dev(s.draft_logits, "bf16"), i32(s.drafts),
                                          s.temperature, s.seed, s.offset, workspace=fill.cuda())
        torch.cuda.synchronize()
        r_acc, r_toks = oracle.accept_sample_ref(s.target_logits, s.draft_logits, s.drafts,
                                                 "bf16", s.temperature, s.seed, s.offset)
        np.testing.assert_array_equal(acc.cpu().numpy(), r_acc)
        np.testing.assert_array_equal(toks.cpu().numpy(), r_toks)
    say("[sample] graph replays")
    s0 = ss[3]
    tl, dl = to_dev(s0.target_logits, "bf16"), to_dev(s0.draft_logits, "bf16")
    dr = i32(s0.drafts)
    ws = torch.full((n.value,), 0xA5, dtype=torch.uint8, device="cuda")
    outs = (torch.empty(B, dtype=torch.int32, device="cuda"),
            torch.empty(B, K, dtype=torch.int32, device="cuda"))
    st = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        gpu_lib.accept_sample(tl, dl, dr, s0.temperature, s0.seed, s0.offset, out=outs,
                              workspace=ws, stream=st)
    for r in range(4):
        s = ss[3 + r]
        tl.copy_(to_dev(s.target_logits, "bf16"))
        dl.copy_(to_dev(s.draft_logits, "bf16"))
        dr.copy_(i32(s.drafts))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        r_acc, r_toks = oracle.accept_sample_ref(s.target_logits, s.draft_logits, s.drafts,
                                                 "bf16", s.temperature, s.seed, s0.offset)
        np.testing.assert_array_equal(outs[0].cpu().numpy(), r_acc, err_msg=f"replay {r}")
        np.testing.assert_array_equal(outs[1].cpu().numpy(), r_toks, err_msg=f"replay {r}")


def test_sample_waits_that_give_up_are_reported(gpu_lib):
    """With the wait limit forced down to one poll from the host, the last race workgroup
    of a sequence may give up waiting for the other chunks' winners: every sequence then
    either matches the oracle or reports accept_len -1 with all tokens -1, and every
    kernel still ends normally.  The default limit gives the oracle's results."""
    s = W.make_sample(np.random.default_rng(31), B=8, K=32, V=152064, dtype="bf16",
                      seed=0x5EED, offset=3)
    r_acc, r_toks = oracle.accept_sample_ref(s.target_logits, s.draft_logits, s.drafts, "bf16",
                                             s.temperature, s.seed, s.offset)
    failed = 0
    try:
        gpu_lib.set_wait_limit(1)
        for rep in range(4):
            say(f"[sample] wait limit 1, call {rep}")
            acc, toks = sample_gpu(gpu_lib, s)
            for b in range(s.B):
                if acc[b] == -1:
                    failed += 1
                    assert (toks[b] == -1).all()
                else:
                    assert acc[b] == r_acc[b]
                    np.testing.assert_array_equal(toks[b], r_toks[b])
    finally:
        gpu_lib.set_wait_limit(1 << 18)
    say(f"  sequences reporting a wait that gave up: {failed} of {4 * s.B}")
    assert_sample(gpu_lib, s, "default wait limit")


def test_sample_workspace_shape_change(gpu_lib):
    """A workspace first used by a large call and then by a smaller one with more
    sequences: the race's winner slots (which the last chunk of each sequence waits on)
    must not inherit the earlier call's winners."""
    rng = np.random.default_rng(12)
    for i, (B, K, V) in enumerate([(1, 32, 60000), (16, 8, 1000), (2, 4, 30000), (24, 3, 500)]):
        s = W.make_sample(rng, B=B, K=K, V=V, dtype="bf16", seed=5, offset=i)
        say(f"[sample] shape change {i}: B={B} K={K} V={V}")
        assert_sample(gpu_lib, s, f"shape{i}")


# ------------------------------------------------------------------------- commit
@pytest.mark.parametrize("name", ["qwen7b_25k", "batched_paged"])
def test_commit_after_greedy(gpu_lib, name):
    """Device-side cycle close on the acceptance kernel's own outputs, chained over
    several cycles with the context kept on the device: bit-exact against the oracle."""
    g0 = W.make_workload_greedy(name, 0)
    ctx_dev = torch.arange(100, 100 + g0.B, dtype=torch.int32, device="cuda")
    ctx_ref = ctx_dev.cpu().numpy()
    for cycle in range(3):
        g = W.make_workload_greedy(name, cycle)
        say(f"[commit] workload={name} cycle={cycle} B={g.B}")
        acc, toks, _ = gpu_lib.accept_greedy(to_dev(g.logits, g.dtype), i32(g.drafts))
        anchor = gpu_lib.commit(acc, toks, ctx_dev)
        torch.cuda.synchronize()
        ctx_ref, anchor_ref = oracle.commit_ref(ctx_ref, acc.cpu().numpy(), toks.cpu().numpy())
        np.testing.assert_array_equal(ctx_dev.cpu().numpy(), ctx_ref)
        np.testing.assert_array_equal(anchor.cpu().numpy(), anchor_ref)


def test_commit_edges(gpu_lib):
    """accept_len 0 and K-1, K = 1, and a batch spanning several workgroups."""
    rng = np.random.default_rng(77)
    for B, K in [(1, 1), (3, 16), (1000, 8)]:
        acc = rng.integers(0, K, B).astype(np.int32)
        acc[0] = 0
        acc[-1] = K - 1
        toks = rng.integers(0, 152064, (B, K)).astype(np.int32)
        ctx = rng.integers(0, 30000, B).astype(np.int32)
        say(f"[commit] edges B={B} K={K}")
        ctx_dev = i32(ctx)
        anchor = gpu_lib.commit(i32(acc), i32(toks), ctx_dev)
        torch.cuda.synchronize()
        r_ctx, r_anchor = oracle.commit_ref(ctx, acc, toks)
        np.testing.assert_array_equal(ctx_dev.cpu().numpy(), r_ctx)
        np.testing.assert_array_equal(anchor.cpu().numpy(), r_anchor)


def test_sample_a_thousand_sequence_cycles(gpu_lib):
    """1,024 seeded sequence-cycles of the 72B block shape (K = 32) on a smaller
    vocabulary: every accept length and token bit-exact; the smallest distance of any
    uniform from its threshold and the smallest race gap are reported."""
    rng = np.random.default_rng(4242)
    margins, gaps, accepted = [], [], 0
    for off in range(128):
        s = W.make_sample(rng, B=8, K=32, V=3000, dtype="bf16", seed=0x5EED, offset=off)
        if off % 32 == 0:
            say(f"[sample] thousand cycles: offset {off}")
        acc, m, gp = assert_sample(gpu_lib, s, f"offset {off}")
        margins.append(m)
        gaps.append(gp)
        accepted += int(acc.sum())
    say(f"  accepted drafts {accepted} over 1024 sequence-cycles; smallest margin "
        f"{min(margins):.2e}, smallest race gap {min(gaps):.2e}")
    assert accepted > 0


# ------------------------------------------------------------------ un-planted inputs
def _drafts_following(rng, t, V):
    """Drafts that copy the oracle's greedy tokens t [B][K] for a Geometric(0.25) prefix,
    then differ once, then are uniform (test-side; the argmax comes from the oracle)."""
    B, K = t.shape
    L = np.minimum(rng.geometric(0.25, size=B) - 1, K - 1)
    drafts = rng.integers(0, V, size=(B, K - 1)).astype(np.int32)
    for b in range(B):
        n = int(L[b])
        drafts[b, :n] = t[b, :n]
        if n < K - 1 and V > 1:
            o = int(rng.integers(0, V - 1))
            drafts[b, n] = o if o < t[b, n] else o + 1
    return drafts, L


@pytest.mark.parametrize("B,K,sign", [(1, 16, "mixed"), (8, 16, "mixed"), (4, 16, "negative"),
                                      (2, 32, "negative")])
def test_greedy_unplanted_full_vocabulary(gpu_lib, B, K, sign):
    """Plain N(0, 3) bf16 rows over the full 152,064-token vocabulary, nothing planted:
    the natural bf16 ties (a few percent of rows) and, for "negative", rows whose every
    logit (and so the maximum) is negative -- the ordering of negative keys."""
    V = 152064
    rng = np.random.default_rng([77, B, K, len(sign)])
    x = rng.standard_normal(size=(B, K, V), dtype=np.float32) * np.float32(3.0)
    if sign == "negative":
        x = -np.abs(x) - np.float32(0.25)
    logits = W.bf16_bits(x)
    _, _, t = oracle.accept_greedy_ref(logits, np.zeros((B, K - 1), np.int32), "bf16")
    drafts, L = _drafts_following(rng, t, V)
    xs = W.bf16_bits_to_f32(logits)
    ties = int(((xs == xs.max(axis=-1, keepdims=True)).sum(axis=-1) > 1).sum())
    say(f"[greedy] unplanted B={B} K={K} V={V} {sign}: rows with a tied maximum {ties}/{B * K}")
    acc = assert_greedy(gpu_lib, logits, drafts, "bf16", f"unplanted {sign}")
    np.testing.assert_array_equal(acc, L)
    if sign == "negative":
        assert (xs.max(axis=-1) < 0).all()


def test_greedy_unplanted_ties_are_common(gpu_lib):
    """Rows built to hold their maximum several times at scattered indices, in f32 and
    bf16, over the full vocabulary: the lowest index must win."""
    V, K = 152064, 16
    rng = np.random.default_rng(4321)
    x = rng.standard_normal(size=(2, K, V), dtype=np.float32) * np.float32(3.0)
    for b in range(2):
        for i in range(K):
            idx = rng.choice(V, size=4, replace=False)
            if i % 2:                               # a positive maximum held 4 times
                x[b, i, idx] = 30.0
            else:                                   # every logit negative, maximum -0.75
                x[b, i] = -np.abs(x[b, i]) - 1.0
                x[b, i, idx] = -0.75
    for dtype in ("f32", "bf16"):
        logits = x if dtype == "f32" else W.bf16_bits(x)
        _, _, t = oracle.accept_greedy_ref(logits, np.zeros((2, K - 1), np.int32), dtype)
        drafts, L = _drafts_following(rng, t, V)
        say(f"[greedy] planted multi-ties {dtype}")
        acc = assert_greedy(gpu_lib, logits, drafts, dtype, f"multi-ties {dtype}")
        np.testing.assert_array_equal(acc, L)


# ------------------------------------------------------------------ 72B sampling at scale
GOLDEN_72B = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                          "sample_72b_1024.json")


def test_sample_72b_thousand_sequence_cycles(gpu_lib):
    """1,024 sequence-cycles of the 72B sampling shape at the full vocabulary (8 sequences
    x 128 Philox offsets): every accept length and drawn token bit-exact with the oracle's
    verdicts, which tests/golden/make_sample_72b.py stored (oracle calls only); the inputs
    are regenerated and checked against the stored digest, and four offsets are also
    re-run through the oracle live.  The smallest |u - threshold| and relative race gap
    over all 1,024 are printed."""
    import make_sample_72b as G
    with open(GOLDEN_72B) as fh:
        gold = json.load(fh)
    s = G.inputs()
    assert G.digest(s) == gold["input_digest"], "the input generator changed"
    tl = to_dev(s.target_logits, s.dtype)
    dl = to_dev(s.draft_logits, s.dtype)
    dr = i32(s.drafts)
    accepted, margins, gaps = 0, [], []
    for off in range(G.OFFSETS):
        if off % 32 == 0:
            say(f"[sample] 72B x 8 sequences, offsets {off}..{off + 31}")
        acc, toks = gpu_lib.accept_sample(tl, dl, dr, s.temperature, s.seed, off)
        torch.cuda.synchronize()
        acc, toks = acc.cpu().numpy(), toks.cpu().numpy()
        g = gold["offsets"][str(off)]
        np.testing.assert_array_equal(acc, g["accept_len"], err_msg=f"offset {off}")
        for b in range(s.B):
            a = int(acc[b])
            assert list(toks[b, :a]) == list(s.drafts[b, :a]), (off, b)
            assert toks[b, a] == g["token"][b], (off, b, toks[b, a], g["token"][b],
                                                 g["margin"][b], g["race_gap"][b])
            assert (toks[b, a + 1:] == -1).all()
        accepted += int(acc.sum())
        margins += g["margin"]
        gaps += g["race_gap"]
        if off % 32 == 5:                          # the oracle live, on the same inputs
            r_acc, r_toks = oracle.accept_sample_ref(s.target_logits, s.draft_logits,
                                                     s.drafts, s.dtype, s.temperature,
                                                     s.seed, off)
            np.testing.assert_array_equal(acc, r_acc)
            np.testing.assert_array_equal(toks, r_toks)
    say(f"  1024 sequence-cycles: accepted drafts {accepted}; smallest |u - threshold| "
        f"{min(margins):.3e}, smallest relative race gap {min(gaps):.3e}")


def test_sample_masked_vocabulary(gpu_lib):
    """-inf logits: whole 8192-entry chunks of the vocabulary masked in the target and
    the draft rows (and a stretch not aligned to chunks), a draft the target gives
    probability 0 (always rejected) and one the draft gives probability 0 (always
    accepted): bit-exact with the oracle, and nothing masked is ever drawn."""
    V, K, B = 40000, 8, 6
    rng = np.random.default_rng(606)
    for off in range(8):
        s = W.make_sample(rng, B=B, K=K, V=V, dtype="bf16", seed=9, offset=off)
        t = W.bf16_bits_to_f32(s.target_logits)
        d = W.bf16_bits_to_f32(s.draft_logits)
        t[:, :, 8192:24576] = -np.inf               # two whole normaliser chunks
        d[:, :, 8192:16384] = -np.inf
        t[:, :, 30001:31234] = -np.inf              # not chunk-aligned
        s.drafts[0, 0] = 9000                       # p = 0: rejected at k = 1
        s.drafts[1, 2] = 12000                      # p = 0 at k = 3
        t[2, 1, 12000] = 5.0                        # p > 0 while q = 0 at k = 2 ...
        s.drafts[2, 1] = 12000                      # ... so it is accepted
        s.target_logits = W.bf16_bits(t)
        s.draft_logits = W.bf16_bits(d)
        say(f"[sample] masked vocabulary offset={off}")
        acc, toks = sample_gpu(gpu_lib, s)
        assert_sample(gpu_lib, s, f"masked/{off}")
        assert acc[0] == 0
        tk = toks[np.arange(B), acc]
        assert not (((tk >= 8192) & (tk < 24576)) | ((tk >= 30001) & (tk < 31234))).any()


def test_sample_many_chunk_partials(gpu_lib):
    """K = 64 over a 300,000-token vocabulary: more chunk partials per sequence than a race
    workgroup folds itself, so the separate normaliser pass runs."""
    rng = np.random.default_rng(3030)
    s = W.make_sample(rng, B=1, K=64, V=300000, dtype="bf16", seed=17, offset=0)
    for off in range(3):
        s.offset = off
        say(f"[sample] K=64 V=300000 offset={off}")
        assert_sample(gpu_lib, s, f"wide/{off}")
