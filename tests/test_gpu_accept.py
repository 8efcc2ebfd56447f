"""GPU parity of sv_accept_greedy / sv_accept_sample against the oracle: bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import i32, say, to_dev

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


def test_sample_workspace_shape_change(gpu_lib):
    """A workspace first used by a large call and then by a smaller one with more
    sequences: the arrival counters must not inherit the earlier call's partial sums."""
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
