"""Upload helpers for the GPU parity tests (seeded numpy inputs -> device tensors)."""
import sys

import numpy as np
import torch

import oracle


def say(*a):
    """Name the case before a GPU step, flushed, so a failing run shows where it was."""
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a, dtype: str):
    """Stored numpy array (bf16 as uint16 bits) -> device tensor of that dtype."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).cuda()
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    raise ValueError(dtype)


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def upload_verify(inp):
    return dict(q=to_dev(inp.q, inp.dtype), k_cache=to_dev(inp.k_cache, inp.dtype),
                v_cache=to_dev(inp.v_cache, inp.dtype), page_table=i32(inp.page_table),
                ctx_lens=i32(inp.ctx_lens))


def attn_tolerance(dtype):
    """(abs, rel-to-slice-max, lse) bounds: bf16/f16 inputs follow max-abs 2e-2 and rel
    1e-2; fp32 inputs rel 1e-4."""
    if dtype == "f32":
        return 1e-4, 1e-4, 1e-5
    return 2e-2, 1e-2, 1e-3


def check_attention(got_out, got_lse, ref_out, ref_lse, dtype, where=""):
    """Element-by-element comparison with the oracle, per (b, head) slice."""
    a_tol, r_tol, l_tol = attn_tolerance(dtype)
    g = got_out.float().cpu().numpy().astype(np.float64)
    diff = np.abs(g - ref_out)
    assert np.isfinite(g).all(), f"{where}: non-finite output"
    worst = diff.max()
    assert worst <= a_tol, f"{where}: max |d| {worst:.3e} > {a_tol}"
    # per (b, head) slice: max |d| <= r_tol * max |ref| over that slice
    slice_max = np.abs(ref_out).max(axis=(1, 3))          # [B][Hq]
    slice_err = diff.max(axis=(1, 3))
    ratio = (slice_err / np.maximum(slice_max, 1e-30)).max()
    assert ratio <= r_tol, f"{where}: slice-relative error {ratio:.3e} > {r_tol}"
    if got_lse is not None:
        dl = np.abs(got_lse.cpu().numpy().astype(np.float64) - ref_lse).max()
        assert dl <= l_tol, f"{where}: max |d lse| {dl:.3e} > {l_tol}"
    return worst, ratio
