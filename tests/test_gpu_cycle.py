"""Device-resident verification cycles: append the block's K/V at the device-side context
length, verify, accept, commit -- chained over cycles with the state never leaving the
device -- against the oracle's own chain of the same steps."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import check_attention, i32, say, to_dev

pytestmark = pytest.mark.gpu


def test_chained_cycles_stay_in_step_with_the_oracle(gpu_lib):
    rng = np.random.default_rng(2024)
    B, K, Hq, Hkv, D, P, V = 3, 16, 28, 4, 128, 16, 5000
    cycles = 4
    ctx0 = np.array([300, 1000, 57], dtype=np.int32)
    cap = int(ctx0.max()) + (cycles + 1) * K            # room for every cycle's block
    # a cache with capacity `cap` per sequence: the workload generator fills the first
    # ctx0 + K tokens; the rest of each sequence's pages is written by the appends
    inp = W.make_verify(rng, B=B, K=K, Hq=Hq, Hkv=Hkv, D=D, ctx_lens=[cap - K] * B, P=P,
                        dtype="bf16", shuffle=True)
    kc_ref, vc_ref = inp.k_cache.copy(), inp.v_cache.copy()
    kc, vc = to_dev(kc_ref, "bf16"), to_dev(vc_ref, "bf16")
    pt = i32(inp.page_table)
    ctx_dev = i32(ctx0)
    ctx_ref = ctx0.copy()
    for c in range(cycles):
        say(f"[cycle] {c}: ctx {ctx_ref.tolist()}")
        k_new = W.bf16_bits(rng.standard_normal((B, K, Hkv, D), dtype=np.float32))
        v_new = W.bf16_bits(rng.standard_normal((B, K, Hkv, D), dtype=np.float32))
        q = W.bf16_bits(rng.standard_normal((B, K, Hq, D), dtype=np.float32))
        # append at the device-side context length, then verify over ctx + block
        gpu_lib.kv_append(to_dev(k_new, "bf16"), to_dev(v_new, "bf16"), ctx_dev, pt, kc, vc)
        out, lse = gpu_lib.verify_attention(to_dev(q, "bf16"), kc, vc, pt, ctx_dev,
                                            max_ctx=cap - K)
        kc_ref, vc_ref = oracle.kv_append_ref(kc_ref, vc_ref, inp.page_table, ctx_ref, k_new, v_new)
        step = W.VerifyInputs(B, K, Hq, Hkv, D, P, "bf16", q, kc_ref, vc_ref, inp.page_table,
                              ctx_ref.copy(), W.causal_mask(K))
        ref_out, ref_lse = oracle.verify_attention_ref(step)
        torch.cuda.synchronize()
        check_attention(out, lse, ref_out, ref_lse, "bf16", f"cycle {c}")
        # accept on planted logits, then close the cycle on the device
        g = W.make_greedy(rng, B=B, K=K, V=V, dtype="bf16")
        acc, toks, _ = gpu_lib.accept_greedy(to_dev(g.logits, "bf16"), i32(g.drafts))
        anchor = gpu_lib.commit(acc, toks, ctx_dev)
        torch.cuda.synchronize()
        r_acc, r_toks, _ = oracle.accept_greedy_ref(g.logits, g.drafts, "bf16")
        ctx_ref, r_anchor = oracle.commit_ref(ctx_ref, r_acc, r_toks)
        np.testing.assert_array_equal(acc.cpu().numpy(), r_acc)
        np.testing.assert_array_equal(anchor.cpu().numpy(), r_anchor)
        np.testing.assert_array_equal(ctx_dev.cpu().numpy(), ctx_ref)
    # the caches hold exactly the oracle's appended rows
    np.testing.assert_array_equal(kc.view(torch.int16).cpu().numpy().view(np.uint16), kc_ref)
    np.testing.assert_array_equal(vc.view(torch.int16).cpu().numpy().view(np.uint16), vc_ref)
