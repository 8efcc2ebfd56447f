"""GPU parity of sv_verify_attention against the float64 oracle (needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import check_attention, i32, say, to_dev, upload_verify

pytestmark = pytest.mark.gpu


def run(sv, inp, split_keys=0, max_ctx=None, hint=True):
    d = upload_verify(inp)
    mc = int(inp.ctx_lens.max()) if max_ctx is None else max_ctx
    out, lse = sv.verify_attention(d["q"], d["k_cache"], d["v_cache"], d["page_table"],
                                   d["ctx_lens"], max_ctx=mc, block_mask=inp.mask,
                                   split_keys=split_keys,
                                   sum_ctx_hint=int(inp.ctx_lens.sum()) if hint else 0)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("name", ["tiny_fp32", "qwen7b_25k", "batched_paged", "qwen72b_sampling",
                                  "vflash_drafter"])
def test_named_workloads_full_size(gpu_lib, name):
    """The workloads at their full sizes, in the launch configuration the bench uses."""
    inp = W.make_workload_verify(name)
    say(f"[attention] workload={name} B={inp.B} K={inp.K} Hq={inp.Hq} Hkv={inp.Hkv} "
        f"D={inp.D} ctx={list(inp.ctx_lens)} dtype={inp.dtype}")
    out, lse = run(gpu_lib, inp)
    ref_out, ref_lse = oracle.verify_attention_ref(inp)
    worst, ratio = check_attention(out, lse, ref_out, ref_lse, inp.dtype, name)
    say(f"  max|d|={worst:.2e} slice-rel={ratio:.2e}")


CASES = [
    # dtype, D, P, Hq, Hkv, K, ctx, split_keys, mask, shuffle
    ("bf16", 128, 16, 28, 4, 16, [1000], 0, "causal", False),
    ("bf16", 128, 16, 28, 4, 16, [1000], 64, "causal", True),     # many splits
    ("bf16", 128, 16, 28, 4, 16, [777], 16, "causal", True),      # 16-key splits, ragged tile
    ("bf16", 128, 32, 8, 8, 5, [333, 70], 96, "ones", True),      # G=1, 3 pages per split
    ("bf16", 64, 16, 64, 64, 5, [64], 0, "ones", False),          # SAR-like: d 64, K 5
    ("bf16", 128, 256, 14, 2, 9, [3001], 0, "random", True),      # big pages
    ("bf16", 128, 64, 64, 8, 32, [2500], 0, "causal", False),     # 256 rows: 2 row blocks
    ("bf16", 64, 16, 16, 2, 3, [0], 0, "causal", False),          # empty context
    ("bf16", 128, 16, 4, 4, 1, [90], 0, "causal", True),          # single block row
    ("bf16", 128, 16, 2, 1, 64, [513], 0, "causal", False),       # K = 64 (max)
    ("f16", 128, 16, 28, 4, 16, [1500, 1, 4097], 0, "causal", True),
    ("f16", 64, 32, 12, 3, 7, [200, 300], 32, "random", True),
    ("f32", 64, 16, 2, 1, 4, [512], 0, "causal", False),
    ("f32", 128, 16, 8, 2, 6, [250, 999], 0, "random", True),
    ("f32", 64, 64, 6, 2, 16, [77], 64, "ones", True),
    # one split per (b, g): the split pass writes the output and lse itself (no merge)
    ("bf16", 128, 16, 28, 4, 16, [40], 0, "causal", True),       # 112 rows, 512 threads
    ("f16", 64, 16, 64, 64, 5, [64, 64, 17], 0, "ones", True),   # 5 rows: 128-thread pair
    ("f32", 64, 16, 4, 2, 4, [30, 0], 0, "random", False),
    ("bf16", 128, 16, 64, 8, 32, [20], 0, "causal", False),      # 256 rows: one 256-row group
    ("f32", 64, 16, 32, 4, 20, [40], 0, "causal", True),         # 160 rows, fp32: two groups of 128
    # at most 32 rows at d 64: the 128-thread workgroup over many splits (then the merge),
    # and a split longer than its 8192-key page-id stage (the 512-thread kernel instead)
    ("bf16", 64, 16, 8, 8, 5, [3000], 0, "causal", True),
    ("f16", 64, 16, 8, 8, 5, [9000], 8256, "ones", True),
]


def _mask(kind, K, rng):
    if kind == "causal":
        return W.causal_mask(K)
    if kind == "ones":
        return W.all_ones_mask(K)
    return np.array([(int(rng.integers(0, 1 << min(K, 62))) | (1 << i)) & ((1 << K) - 1)
                     for i in range(K)], dtype=np.uint64)


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_shapes_and_edges(gpu_lib, case):
    dtype, D, P, Hq, Hkv, K, ctx, split, mk, shuffle = case
    rng = np.random.default_rng(100 + CASES.index(case))
    inp = W.make_verify(rng, B=len(ctx), K=K, Hq=Hq, Hkv=Hkv, D=D, ctx_lens=ctx, P=P,
                        dtype=dtype, shuffle=shuffle, mask=_mask(mk, K, rng))
    say(f"[attention] case={case}")
    out, lse = run(gpu_lib, inp, split_keys=split)
    ref_out, ref_lse = oracle.verify_attention_ref(inp)
    check_attention(out, lse, ref_out, ref_lse, dtype, str(case))


def run_poisoned(sv, inp, split_keys, max_ctx):
    """Like run(), into a workspace filled with 0xFF bytes (NaN as floats): any partial
    of an absent split that the merge failed to ignore would surface in the output."""
    d = upload_verify(inp)
    desc = sv.make_desc(d["q"], d["k_cache"], d["page_table"], max_ctx, 0.0, split_keys, 0)
    ws = torch.full((sv.attention_workspace_bytes(desc),), 255, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d["q"])
    lse = torch.empty(d["q"].shape[:3], dtype=torch.float32, device="cuda")
    sv.verify_attention_into(desc, d["q"], d["k_cache"], d["v_cache"], d["page_table"],
                             d["ctx_lens"], out, lse, sv.mask_array(inp.mask), ws)
    torch.cuda.synchronize()
    return out, lse


def test_max_ctx_above_actual_and_no_hint(gpu_lib):
    """Grid sized for a larger max_ctx than any sequence has (a batch: the context length
    is read first): surplus splits exit early, leaving only empty (m, l) pairs."""
    rng = np.random.default_rng(7)
    inp = W.make_verify(rng, B=3, K=16, Hq=28, Hkv=4, D=128, ctx_lens=[100, 2000, 37], P=16,
                        dtype="bf16", shuffle=True)
    # pad every page-table row so max_ctx = 4000 is addressable; extra entries point at page 0
    need = (4000 + 16 + 15) // 16
    pt = np.zeros((3, need), dtype=np.int32)
    pt[:, :inp.page_table.shape[1]] = np.where(inp.page_table >= 0, inp.page_table, 0)
    inp.page_table = pt
    say("[attention] max_ctx=4000 over ctx [100, 2000, 37], poisoned workspace")
    out, lse = run_poisoned(gpu_lib, inp, split_keys=0, max_ctx=4000)
    ref_out, ref_lse = oracle.verify_attention_ref(inp)
    check_attention(out, lse, ref_out, ref_lse, "bf16", "max_ctx")


def test_single_sequence_surplus_splits(gpu_lib):
    """One sequence (start-up loads issued before the context length is known) with a
    grid sized for max_ctx = 2000 over ctx 300: the surplus splits load, then leave an
    empty (m, l) pair per row; the merge must treat them as absent."""
    rng = np.random.default_rng(8)
    inp = W.make_verify(rng, B=1, K=16, Hq=28, Hkv=4, D=128, ctx_lens=[300], P=16,
                        dtype="bf16", shuffle=True)
    need = (2000 + 16 + 15) // 16
    pt = np.zeros((1, need), dtype=np.int32)
    pt[:, :inp.page_table.shape[1]] = np.where(inp.page_table >= 0, inp.page_table, 0)
    inp.page_table = pt
    say("[attention] B=1 max_ctx=2000 over ctx [300], 64-key splits, poisoned workspace")
    out, lse = run_poisoned(gpu_lib, inp, split_keys=64, max_ctx=2000)
    ref_out, ref_lse = oracle.verify_attention_ref(inp)
    check_attention(out, lse, ref_out, ref_lse, "bf16", "surplus")


def test_more_splits_than_one_merge_round(gpu_lib):
    """126 splits of 16 keys: each merge wave folds two rounds of 8 splits; the last
    split holds only block keys 7..15, which rows 0..6 cannot see (l = 0 there)."""
    rng = np.random.default_rng(9)
    inp = W.make_verify(rng, B=1, K=16, Hq=28, Hkv=4, D=128, ctx_lens=[1993], P=16,
                        dtype="bf16", shuffle=True)
    say("[attention] ctx 1993, 16-key splits (126 splits), poisoned workspace")
    out, lse = run_poisoned(gpu_lib, inp, split_keys=16, max_ctx=1993)
    ref_out, ref_lse = oracle.verify_attention_ref(inp)
    check_attention(out, lse, ref_out, ref_lse, "bf16", "two merge rounds")


def test_deterministic_repeats(gpu_lib):
    """100 identical calls give bit-identical outputs (every reduction has a fixed order)."""
    inp = W.make_verify(np.random.default_rng(3), B=2, K=16, Hq=28, Hkv=4, D=128,
                        ctx_lens=[3000, 1234], P=16, dtype="bf16", shuffle=True)
    d = upload_verify(inp)
    say("[attention] determinism x100")
    first = None
    for _ in range(100):
        out, lse = gpu_lib.verify_attention(d["q"], d["k_cache"], d["v_cache"], d["page_table"],
                                            d["ctx_lens"], max_ctx=3000)
        if first is None:
            first = (out.clone(), lse.clone())
        else:
            assert torch.equal(out, first[0]) and torch.equal(lse, first[1])


def test_checker_rejects_mutants(gpu_lib):
    """The parity check is sharp: a zero output, a dropped split and a shifted mask fail.
    (On a short context: one extra key among 25k moves outputs far less than the
    tolerance, so mask mistakes are caught by the short-context cases.)"""
    inp = W.make_verify(np.random.default_rng(4), B=1, K=16, Hq=28, Hkv=4, D=128,
                        ctx_lens=[20], P=16, dtype="bf16")
    say("[attention] mutants")
    out, lse = run(gpu_lib, inp, split_keys=16)
    ref_out, ref_lse = oracle.verify_attention_ref(inp)
    check_attention(out, lse, ref_out, ref_lse, "bf16", "base")
    with pytest.raises(AssertionError):
        check_attention(torch.zeros_like(out), None, ref_out, ref_lse, "bf16", "zero")
    # the oracle over a cache missing its first 16 keys (one dropped split)
    dropped = W.VerifyInputs(**{**inp.__dict__})
    dropped.k_cache = inp.k_cache.copy()
    dropped.k_cache[:1] = 0
    dropped.v_cache = inp.v_cache.copy()
    dropped.v_cache[:1] = 0
    d_out, d_lse = oracle.verify_attention_ref(dropped)
    with pytest.raises(AssertionError):
        check_attention(out, lse, d_out, d_lse, "bf16", "dropped split")
    shifted = W.VerifyInputs(**{**inp.__dict__})
    shifted.mask = np.array([(1 << (i + 2)) - 1 if i < 15 else (1 << 16) - 1 for i in range(16)],
                            dtype=np.uint64)
    s_out, s_lse = oracle.verify_attention_ref(shifted)
    with pytest.raises(AssertionError):
        check_attention(out, lse, s_out, s_lse, "bf16", "off-by-one mask")


def test_kv_append_then_verify(gpu_lib):
    """The block's rows written with sv_kv_append land where the oracle layout says."""
    rng = np.random.default_rng(8)
    inp = W.make_verify(rng, B=3, K=16, Hq=28, Hkv=4, D=128, ctx_lens=[500, 37, 1200], P=16,
                        dtype="bf16", shuffle=True)
    new_k = W.bf16_bits(rng.standard_normal((3, 16, 4, 128), dtype=np.float32))
    new_v = W.bf16_bits(rng.standard_normal((3, 16, 4, 128), dtype=np.float32))
    kc_ref, vc_ref = oracle.kv_append_ref(inp.k_cache, inp.v_cache, inp.page_table,
                                          inp.ctx_lens, new_k, new_v)
    d = upload_verify(inp)
    say("[kv_append] B=3 n=16")
    gpu_lib.kv_append(to_dev(new_k, "bf16"), to_dev(new_v, "bf16"), i32(inp.ctx_lens),
                      d["page_table"], d["k_cache"], d["v_cache"])
    torch.cuda.synchronize()
    got_k = d["k_cache"].view(torch.int16).cpu().numpy().view(np.uint16)
    got_v = d["v_cache"].view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got_k, kc_ref)
    np.testing.assert_array_equal(got_v, vc_ref)
