"""GPU parity of sv_accept_sample_tree (sampling verification of a draft tree) against the
float64 oracle: accept lengths, tokens and paths bit-exact; on a chain it equals
sv_accept_sample."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import i32, say, to_dev

pytestmark = pytest.mark.gpu


def tree_gpu(sv, ts, offset=None):
    off = ts.offset if offset is None else offset
    acc, toks, path = sv.accept_sample_tree(to_dev(ts.target_logits, ts.dtype),
                                            to_dev(ts.draft_logits, ts.dtype), ts.parents,
                                            i32(ts.tokens), ts.temperature, ts.seed, off)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), toks.cpu().numpy(), path.cpu().numpy()


def assert_tree(sv, ts, where, offset=None):
    off = ts.offset if offset is None else offset
    acc, toks, path = tree_gpu(sv, ts, off)
    r_acc, r_toks, r_path = oracle.accept_sample_tree_ref(ts.target_logits, ts.draft_logits,
                                                          ts.parents, ts.tokens, ts.dtype,
                                                          ts.temperature, ts.seed, off)
    np.testing.assert_array_equal(acc, r_acc, err_msg=f"{where}: accept_len")
    np.testing.assert_array_equal(path, r_path, err_msg=f"{where}: path")
    np.testing.assert_array_equal(toks, r_toks, err_msg=f"{where}: out_tokens")
    return acc


def test_tree60_workload(gpu_lib):
    """The static Tree-60 (61 nodes, the anchor with 10 children) over the full 152,064-token
    vocabulary: 8 cycles of fresh inputs (2 sequences each, Philox offset = cycle), six at
    T = 1 and two at T = 2.5; most tests reject, so the residual chains run deep."""
    depths = []
    for cyc in range(8):
        ts = W.make_workload_tree_sample(cycle=cyc, B=2)
        if cyc >= 6:
            ts.temperature = 2.5
        say(f"[tree sample] Tree-60 cycle={cyc} T={ts.temperature}")
        depths += [int(a) for a in assert_tree(gpu_lib, ts, f"tree60/{cyc}")]
    say(f"  accepted depths {depths}")
    assert max(depths) > 0 and min(depths) < max(depths)


def test_tree60_one_sequence_against_batch(gpu_lib):
    """Tree-60 at full vocabulary for one sequence (its residual passes 2-9 run as one
    launch whose workgroups keep the residual rows in registers and wait on each other's
    partial sums) against the oracle and, bit for bit, against the same sequence inside a
    batch of two (one launch per pass there): 4 cycles, T = 1 and 2.5."""
    from dataclasses import replace
    for cyc in range(4):
        ts2 = W.make_workload_tree_sample(cycle=10 + cyc, B=2)
        if cyc >= 2:
            ts2.temperature = 2.5
        ts1 = replace(ts2, B=1, target_logits=ts2.target_logits[:1],
                      draft_logits=ts2.draft_logits[:1], tokens=ts2.tokens[:1])
        say(f"[tree sample] Tree-60 one sequence, cycle={10 + cyc} T={ts2.temperature}")
        acc1 = assert_tree(gpu_lib, ts1, f"tree60 B=1/{cyc}")
        acc2, toks2, path2 = tree_gpu(gpu_lib, ts2)
        _, toks1, path1 = tree_gpu(gpu_lib, ts1)
        assert acc1[0] == acc2[0]
        np.testing.assert_array_equal(toks1[0], toks2[0])
        np.testing.assert_array_equal(path1[0], path2[0])


@pytest.mark.parametrize("V,dtype,T", [(152064, "bf16", 1.0), (3001, "f32", 0.7)])
def test_chain_topology_equals_chain_call(gpu_lib, V, dtype, T):
    """A chain through the tree call returns exactly what sv_accept_sample returns."""
    rng = np.random.default_rng(V)
    s = W.make_sample(rng, B=3, K=16, V=V, dtype=dtype, temperature=T, seed=41, offset=0)
    parents = np.arange(15, dtype=np.int32)
    tl, dl, dr = to_dev(s.target_logits, dtype), to_dev(s.draft_logits, dtype), i32(s.drafts)
    for off in range(6):
        say(f"[tree sample] chain V={V} offset={off}")
        a1, t1 = gpu_lib.accept_sample(tl, dl, dr, T, 41, off)
        a2, t2, path = gpu_lib.accept_sample_tree(tl, dl, parents, dr, T, 41, off)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(a1.cpu().numpy(), a2.cpu().numpy())
        np.testing.assert_array_equal(t1.cpu().numpy(), t2.cpu().numpy())
        a = a2.cpu().numpy()
        p = path.cpu().numpy()
        for b in range(3):
            assert list(p[b, :a[b] + 1]) == list(range(a[b] + 1))


@pytest.mark.parametrize("shape", ["star", "random", "binary", "deep"])
def test_tree_shapes_many_offsets(gpu_lib, shape):
    """Small vocabularies, 8 sequences x 24 offsets per tree shape: a star (every node under
    the anchor), a random tree, a binary tree, and a long chain with side branches."""
    rng = np.random.default_rng(len(shape) * 31)
    if shape == "star":
        parents = np.zeros(20, np.int32)
    elif shape == "random":
        parents = np.array([int(rng.integers(0, i)) for i in range(1, 40)], np.int32)
    elif shape == "binary":
        parents = np.array([(i - 1) // 2 for i in range(1, 31)], np.int32)
    else:
        parents = np.array([max(0, i - 1 - (i % 3 == 0)) for i in range(1, 64)], np.int32)
    ts = W.make_tree_sample(rng, B=8, V=2000, parents=parents, dtype="bf16", noise=0.7)
    total = 0
    for off in range(24):
        if off % 8 == 0:
            say(f"[tree sample] {shape} K={len(parents) + 1} offset={off}")
        total += int(assert_tree(gpu_lib, ts, f"{shape}/{off}", off).sum())
    assert total > 0


def test_masked_vocabulary_and_invalid_tokens(gpu_lib):
    """-inf stretches in target and draft rows, tokens outside the vocabulary, fp32 logits."""
    rng = np.random.default_rng(5)
    parents = np.array([0, 0, 0, 1, 1, 2, 4], np.int32)
    ts = W.make_tree_sample(rng, B=6, V=20000, parents=parents, dtype="f32")
    ts.target_logits[:, :, 8192:12000] = -np.inf
    ts.draft_logits[:, :, 16384:20000] = -np.inf
    ts.tokens[0, 0] = -5
    ts.tokens[1, 1] = 20000
    ts.tokens[2, 0] = 9000                        # masked for the target: never accepted
    for off in range(10):
        say(f"[tree sample] masked offset={off}")
        acc = assert_tree(gpu_lib, ts, f"masked/{off}", off)
        assert acc[2] == 0 or tree_gpu(gpu_lib, ts, off)[2][2, 1] != 1


def test_workspace_garbage_and_graph_replays(gpu_lib):
    """The single-launch residual passes and the race's last workgroup wait on slots that
    the first launch of every call empties: calls on workspaces filled with 0xFF bytes,
    with random bytes and with the empty-slot pattern itself match the oracle, and one
    call captured in a HIP graph and replayed four times, with new logits copied in
    eagerly between replays, matches the oracle on every replay."""
    import ctypes
    parents = W.make_tree_topology(np.random.default_rng(21))
    B, K, V = 3, len(parents) + 1, 9000
    n = ctypes.c_size_t()
    assert gpu_lib.load().sv_accept_sample_tree_workspace(B, K, V, ctypes.byref(n)) == 0
    tss = [W.make_tree_sample(np.random.default_rng(800 + i), B=B, V=V, parents=parents,
                              dtype="bf16", offset=i) for i in range(7)]
    gen = torch.Generator(device="cpu").manual_seed(7)
    empty = np.frombuffer(np.array([0x7FF5A5A5A5A5A5A5], np.uint64).tobytes(), np.uint8)
    fills = [torch.full((n.value,), 0xFF, dtype=torch.uint8),
             torch.randint(0, 256, (n.value,), dtype=torch.uint8, generator=gen),
             torch.from_numpy(np.resize(empty, n.value).copy())]

    def ref(ts, off):
        return oracle.accept_sample_tree_ref(ts.target_logits, ts.draft_logits, ts.parents,
                                             ts.tokens, ts.dtype, ts.temperature, ts.seed, off)
    for i, fill in enumerate(fills):
        say(f"[tree sample] workspace fill {i}")
        ts = tss[i]
        acc, toks, path = gpu_lib.accept_sample_tree(
            to_dev(ts.target_logits, "bf16"), to_dev(ts.draft_logits, "bf16"), ts.parents,
            i32(ts.tokens), ts.temperature, ts.seed, ts.offset, workspace=fill.cuda())
        torch.cuda.synchronize()
        r_acc, r_toks, r_path = ref(ts, ts.offset)
        np.testing.assert_array_equal(acc.cpu().numpy(), r_acc)
        np.testing.assert_array_equal(path.cpu().numpy(), r_path)
        np.testing.assert_array_equal(toks.cpu().numpy(), r_toks)
    say("[tree sample] graph replays")
    t0 = tss[3]
    tl, dl = to_dev(t0.target_logits, "bf16"), to_dev(t0.draft_logits, "bf16")
    tk = i32(t0.tokens)
    ws = torch.full((n.value,), 0xA5, dtype=torch.uint8, device="cuda")
    outs = (torch.empty(B, dtype=torch.int32, device="cuda"),
            torch.empty(B, K, dtype=torch.int32, device="cuda"),
            torch.empty(B, K, dtype=torch.int32, device="cuda"))
    st = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        gpu_lib.accept_sample_tree(tl, dl, t0.parents, tk, t0.temperature, t0.seed, t0.offset,
                                   out=outs, workspace=ws, stream=st)
    for r in range(4):
        ts = tss[3 + r]
        tl.copy_(to_dev(ts.target_logits, "bf16"))
        dl.copy_(to_dev(ts.draft_logits, "bf16"))
        tk.copy_(i32(ts.tokens))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        r_acc, r_toks, r_path = ref(ts, t0.offset)
        np.testing.assert_array_equal(outs[0].cpu().numpy(), r_acc, err_msg=f"replay {r}")
        np.testing.assert_array_equal(outs[2].cpu().numpy(), r_path, err_msg=f"replay {r}")
        np.testing.assert_array_equal(outs[1].cpu().numpy(), r_toks, err_msg=f"replay {r}")


def test_random_trees_and_shapes(gpu_lib):
    """160 seeded random cases against the oracle: trees of 2-64 nodes (random parents,
    stars of up to 63 siblings, i.e. 62 dependent residual passes in one launch), batches
    of 1-8, vocabularies of 100-30,000 (odd sizes, sizes just around the 2,048-entry pairs
    of the residual workgroups, sizes not a multiple of 8), bf16 and fp32, T in
    [0.5, 2.5]."""
    rng = np.random.default_rng(2024)
    sizes = [100, 1023, 1024, 2047, 2048, 2049, 4095, 6143, 8191, 12289, 30000]
    for case in range(160):
        K = int(rng.integers(2, 65))
        if case % 5 == 0:
            parents = np.zeros(K - 1, np.int32)                 # a star
        else:
            parents = np.array([rng.integers(0, i + 1) for i in range(K - 1)], np.int32)
        B = int(rng.integers(1, 9))
        V = int(sizes[case % len(sizes)] + (rng.integers(0, 7) if case % 3 == 0 else 0))
        dtype = "f32" if case % 4 == 3 else "bf16"
        T = float(rng.uniform(0.5, 2.5))
        ts = W.make_tree_sample(rng, B=B, V=V, parents=parents, dtype=dtype, temperature=T,
                                noise=float(rng.uniform(0.2, 2.0)), seed=int(rng.integers(1 << 40)),
                                offset=case)
        say(f"[tree sample] random case {case}: B={B} K={K} V={V} {dtype} T={T:.2f}")
        assert_tree(gpu_lib, ts, f"random/{case}")


def test_waits_that_give_up_are_reported(gpu_lib):
    """With the wait limit forced down to one poll from the host, the in-launch waits
    (the single-launch residual passes, the race's last workgroup) may give up: every
    sequence then either matches the oracle or reports accept_len -1 with all outputs -1,
    and every kernel still ends normally.  The default limit gives the oracle's results."""
    ts = W.make_workload_tree_sample(cycle=20, B=1)
    r = oracle.accept_sample_tree_ref(ts.target_logits, ts.draft_logits, ts.parents,
                                      ts.tokens, ts.dtype, ts.temperature, ts.seed, ts.offset)
    failed = 0
    try:
        gpu_lib.set_wait_limit(1)
        for rep in range(6):
            say(f"[tree sample] wait limit 1, call {rep}")
            acc, toks, path = tree_gpu(gpu_lib, ts)
            if acc[0] == -1:
                failed += 1
                assert (toks[0] == -1).all() and (path[0] == -1).all()
            else:
                np.testing.assert_array_equal(acc, r[0])
                np.testing.assert_array_equal(toks, r[1])
                np.testing.assert_array_equal(path, r[2])
    finally:
        gpu_lib.set_wait_limit(1 << 18)
    say(f"  calls reporting a wait that gave up: {failed} of 6")
    assert_tree(gpu_lib, ts, "default wait limit")


def test_concurrent_with_other_streams(gpu_lib):
    """The in-launch waits with other work competing for the compute units: a Tree-60
    sampling call (its residual passes in one launch) on one stream while a 72B-shaped
    chain sampling call and a Tree-60 greedy call run on two other streams, five rounds;
    every result matches the oracle (a wait that gave up would report -1)."""
    ts = W.make_workload_tree_sample(cycle=40, B=1)
    s = W.make_sample(np.random.default_rng(41), B=8, K=32, V=152064, dtype="bf16",
                      seed=0x5EED, offset=9)
    r_tree = oracle.accept_sample_tree_ref(ts.target_logits, ts.draft_logits, ts.parents,
                                           ts.tokens, ts.dtype, ts.temperature, ts.seed,
                                           ts.offset)
    r_acc, r_toks = oracle.accept_sample_ref(s.target_logits, s.draft_logits, s.drafts, "bf16",
                                             s.temperature, s.seed, s.offset)
    g_lg = torch.randn(2, ts.K, ts.V, device="cuda").to(torch.bfloat16)
    g_tok = torch.randint(0, ts.V, (2, ts.K - 1), dtype=torch.int32, device="cuda")
    g_par = torch.from_numpy(np.tile(np.asarray(ts.parents, np.int32), (2, 1))).cuda()
    tl, dl, tk = to_dev(ts.target_logits, "bf16"), to_dev(ts.draft_logits, "bf16"), i32(ts.tokens)
    sl, sd, sr = to_dev(s.target_logits, "bf16"), to_dev(s.draft_logits, "bf16"), i32(s.drafts)
    streams = [torch.cuda.Stream() for _ in range(3)]
    torch.cuda.synchronize()
    for rnd in range(5):
        say(f"[tree sample] concurrent round {rnd}")
        with torch.cuda.stream(streams[1]):
            c_out = gpu_lib.accept_sample(sl, sd, sr, s.temperature, s.seed, s.offset,
                                          stream=streams[1])
        with torch.cuda.stream(streams[2]):
            gpu_lib.accept_greedy_tree(g_lg, g_par, g_tok, stream=streams[2])
        with torch.cuda.stream(streams[0]):
            t_out = gpu_lib.accept_sample_tree(tl, dl, ts.parents, tk, ts.temperature, ts.seed,
                                               ts.offset, stream=streams[0])
        torch.cuda.synchronize()
        np.testing.assert_array_equal(t_out[0].cpu().numpy(), r_tree[0])
        np.testing.assert_array_equal(t_out[1].cpu().numpy(), r_tree[1])
        np.testing.assert_array_equal(t_out[2].cpu().numpy(), r_tree[2])
        np.testing.assert_array_equal(c_out[0].cpu().numpy(), r_acc)
        np.testing.assert_array_equal(c_out[1].cpu().numpy(), r_toks)


def test_deterministic_and_offset_sensitive(gpu_lib):
    ts = W.make_tree_sample(np.random.default_rng(9), B=16, V=5000,
                            parents=W.make_tree_topology(np.random.default_rng(3)), dtype="bf16")
    say("[tree sample] determinism")
    r1 = tree_gpu(gpu_lib, ts, 3)
    r2 = tree_gpu(gpu_lib, ts, 3)
    for x, y in zip(r1, r2):
        np.testing.assert_array_equal(x, y)
    r3 = tree_gpu(gpu_lib, ts, 4)
    assert not all(np.array_equal(x, y) for x, y in zip(r1, r3))
