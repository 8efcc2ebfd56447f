"""GPU parity of sv_latent_compress and the SpecFLASH semi-autoregressive block."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import check_attention, i32, say, to_dev

pytestmark = pytest.mark.gpu

# fp16 output (half-ulp 2^-12 relative), fp16-rounded softmax weights (2^-12 relative
# each, so at most 2^-12 * max|F| in a convex combination) and fp32 accumulation:
# |d| <= 2^-11 * |ref| + 2^-11 * max|F|, with max|F| <= 6 for N(0,1) draws at these sizes.
ATOL, RTOL = 4e-3, 2e-3


def compress_gpu(sv, c, scale=1.0):
    out = sv.latent_compress(to_dev(c.queries, "f16"), to_dev(c.feats, "f16"), scale=scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def check(got, ref, where):
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    worst = (err / bound).max()
    assert worst <= 1.0, f"{where}: error {err.max():.3e} exceeds bound by {worst:.2f}x"
    return err.max()


@pytest.mark.parametrize("C,N", [(64, 576), (36, 324)])
def test_compressor_workload(gpu_lib, C, N):
    p = W.WORKLOADS["compressor_sar"].params
    rng = W.rng_for("compressor_sar", C)
    c = W.make_compress(rng, B=p["B"], C=C, N=N, D=p["D"])
    say(f"[compress] B={c.B} C={C} N={N} D={c.D}")
    got = compress_gpu(gpu_lib, c)
    ref = oracle.latent_compress_ref(c.queries, c.feats)
    say(f"  max|d|={check(got, ref, f'{C}x{N}'):.2e}")


@pytest.mark.parametrize("B,C,N,D,scale", [
    (3, 1, 1, 128, 1.0), (2, 33, 100, 256, 1.0), (5, 64, 1024, 384, 0.5), (1, 17, 70, 4096, 1.0),
    # 256-column out tiles (N > 384, D % 256 == 0): partial query block, ragged last tile
    (2, 40, 500, 512, 1.0), (1, 64, 1024, 768, 1.0),
])
def test_compressor_shapes(gpu_lib, B, C, N, D, scale):
    rng = np.random.default_rng(B * 7 + C)
    c = W.make_compress(rng, B=B, C=C, N=N, D=D, q_std=0.1)
    say(f"[compress] B={B} C={C} N={N} D={D} scale={scale}")
    got = compress_gpu(gpu_lib, c, scale)
    ref = oracle.latent_compress_ref(c.queries, c.feats, scale=scale)
    check(got, ref, f"{B},{C},{N},{D}")


@pytest.mark.parametrize("C,N", [(64, 576), (36, 324)])
def test_sar_block_after_compressor(gpu_lib, C, N):
    """Compressor output + 5 slot rows as the K/V of the semi-autoregressive block:
    5 slot queries, 64 heads x 64, one bidirectional block (all-ones mask), for both
    compressor shapes at full size."""
    p = W.WORKLOADS["compressor_sar"].params
    B, D, S, H, HD = p["B"], p["D"], p["S"], p["H"], p["HD"]
    rng = W.rng_for("compressor_sar", 1000 + C)
    c = W.make_compress(rng, B=B, C=C, N=N, D=D)
    sar = W.make_sar(rng, B=B, S=S, H=H, D=HD)
    P = 16
    pages_per = (C + S + P - 1) // P
    table = np.arange(B * pages_per, dtype=np.int32).reshape(B, pages_per)
    kc = torch.zeros(B * pages_per, H, P, HD, dtype=torch.float16, device="cuda")
    vc = torch.zeros(B * pages_per, H, HD, P, dtype=torch.float16, device="cuda")
    say(f"[sar] C={C} N={N}: compressor -> kv_append -> verify attention")
    fhat = gpu_lib.latent_compress(to_dev(c.queries, "f16"), to_dev(c.feats, "f16"))
    rows = fhat.view(B, C, H, HD)
    t_table = i32(table)
    gpu_lib.kv_append(rows, rows, i32(np.zeros(B)), t_table, kc, vc)
    gpu_lib.kv_append(to_dev(sar.slot_k, "f16"), to_dev(sar.slot_v, "f16"),
                      i32(np.full(B, C)), t_table, kc, vc)
    out, lse = gpu_lib.verify_attention(to_dev(sar.q, "f16"), kc, vc, t_table,
                                        i32(np.full(B, C)), max_ctx=C,
                                        block_mask=W.all_ones_mask(S))
    torch.cuda.synchronize()
    # oracle chain: float64 compressor, stored as fp16 like the pipeline stores it, then
    # the same paged layout and the float64 attention
    fh = oracle.latent_compress_ref(c.queries, c.feats).astype(np.float16).reshape(B, C, H, HD)
    kc_ref = np.zeros((B * pages_per, H, P, HD), dtype=np.float16)
    vc_ref = np.zeros((B * pages_per, H, HD, P), dtype=np.float16)
    kc_ref, vc_ref = oracle.kv_append_ref(kc_ref, vc_ref, table, np.zeros(B), fh, fh)
    kc_ref, vc_ref = oracle.kv_append_ref(kc_ref, vc_ref, table, np.full(B, C), sar.slot_k,
                                          sar.slot_v)
    inp = W.VerifyInputs(B, S, H, H, HD, P, "f16", sar.q, kc_ref, vc_ref, table,
                         np.full(B, C, dtype=np.int32), W.all_ones_mask(S))
    ref_out, ref_lse = oracle.verify_attention_ref(inp)
    check_attention(out, lse, ref_out, ref_lse, "f16", f"sar C={C}")
