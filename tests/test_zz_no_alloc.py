"""GPU check of sv_verify_attention_noalloc (the allocation-free verify attention)
through the C ABI: on two calls in a row -- the 7B 25k-context layer, then a smaller
paged batch -- its outputs equal sv_verify_attention's bit for bit (same kernels, same
plan), and both are within the attention tolerance of the float64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import check_attention, say, upload_verify

pytestmark = pytest.mark.gpu


def _both(sv, inp):
    d = upload_verify(inp)
    desc = sv.make_desc(d["q"], d["k_cache"], d["page_table"], int(inp.ctx_lens.max()), 0.0, 0,
                        int(inp.ctx_lens.sum()))
    causal = np.array_equal(inp.mask, W.causal_mask(inp.K))
    mask = None if causal else sv.mask_array(inp.mask)
    ref_out = torch.empty_like(d["q"])
    ref_lse = torch.empty(d["q"].shape[:3], dtype=torch.float32, device="cuda")
    sv.verify_attention_into(desc, d["q"], d["k_cache"], d["v_cache"], d["page_table"],
                             d["ctx_lens"], ref_out, ref_lse, mask)
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full(d["q"].shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    sv.verify_attention_noalloc_into(desc, d["q"], d["k_cache"], d["v_cache"], d["page_table"],
                                     d["ctx_lens"], out, lse, mask)
    torch.cuda.synchronize()
    return out, lse, ref_out, ref_lse


def test_noalloc_matches_the_workspace_call_twice(gpu_lib):
    cases = [("qwen7b_25k", W.make_workload_verify("qwen7b_25k")),
             ("paged B=3", W.make_verify(np.random.default_rng(5), B=3, K=16, Hq=28, Hkv=4,
                                          D=128, ctx_lens=[700, 1337, 64], P=16, dtype="bf16",
                                          shuffle=True))]
    for name, inp in cases:
        say(f"[noalloc] {name}: B={inp.B} K={inp.K} ctx={list(inp.ctx_lens)}")
        out, lse, ref_out, ref_lse = _both(gpu_lib, inp)
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), name
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), name
        r_out, r_lse = oracle.verify_attention_ref(inp)
        check_attention(out, lse, r_out, r_lse, inp.dtype, f"noalloc {name}")
