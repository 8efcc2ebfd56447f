"""GPU parity of the fused LM head + greedy acceptance against the float64 oracle (needs
an MI355X).  The inputs steer every row to a planted token with a gap of several units
(pinned on the CPU), so the argmax cannot depend on the accumulation precision and the
integer outputs must match bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import i32, say, to_dev

pytestmark = pytest.mark.gpu


def _call(sv, hs, w, drafts, packed):
    """The plain call, or the same over the weight packed once by lm_head_pack."""
    if packed:
        return sv.lm_head_greedy_packed(hs, sv.lm_head_pack(w), w.shape[0], drafts)
    return sv.lm_head_greedy(hs, w, drafts)


def _run(sv, li, packed=False):
    acc, toks, am = _call(sv, to_dev(li.hidden_states, li.dtype), to_dev(li.weight, li.dtype),
                          i32(li.drafts), packed)
    torch.cuda.synchronize()
    r_acc, r_toks, r_am, _ = oracle.lm_head_greedy_ref(li.hidden_states, li.weight, li.drafts,
                                                       li.dtype)
    np.testing.assert_array_equal(am.cpu().numpy(), r_am)
    np.testing.assert_array_equal(acc.cpu().numpy(), r_acc)
    np.testing.assert_array_equal(toks.cpu().numpy(), r_toks)
    return r_acc


@pytest.mark.parametrize("packed", [False, True])
def test_qwen7b_lm_head_full_size(gpu_lib, packed):
    li = W.make_workload_lm_head()
    say(f"[lm head] qwen7b_lmhead B={li.B} K={li.K} hidden={li.hidden} V={li.V} packed={packed}")
    r_acc = _run(gpu_lib, li, packed)
    np.testing.assert_array_equal(r_acc, li.planted_len)


@pytest.mark.parametrize("V,hidden,dtype", [(777, 96, "bf16"), (40, 64, "f16"), (1, 32, "bf16"),
                                            (4096, 256, "bf16")])
def test_pack_layout(gpu_lib, V, hidden, dtype):
    """lm_head_pack against the tile layout written out with numpy: pad the rows to a
    multiple of 32 with zeros, view W as [unit][half][row j][chunk q][group g][8] and
    store it as [unit][q][half][g][j][8]; bit for bit."""
    rng = np.random.default_rng([V, hidden])
    w = rng.standard_normal((V, hidden)).astype(np.float32)
    wd = torch.from_numpy(w).to("cuda").to(torch.bfloat16 if dtype == "bf16" else torch.float16)
    say(f"[lm head pack] V={V} hidden={hidden} {dtype}")
    packed = gpu_lib.lm_head_pack(wd)
    torch.cuda.synchronize()
    bits = wd.view(torch.int16).cpu().numpy()
    U, Q = (V + 31) // 32, hidden // 32
    pad = np.zeros((U * 32, hidden), dtype=np.int16)
    pad[:V] = bits
    want = pad.reshape(U, 2, 16, Q, 4, 8).transpose(0, 3, 1, 4, 2, 5).reshape(-1)
    np.testing.assert_array_equal(packed.view(torch.int16).cpu().numpy(), want)


@pytest.mark.parametrize("B,K,hidden,V,dtype", [
    (1, 16, 512, 1000, "bf16"),
    (2, 8, 256, 777, "bf16"),        # ragged last workgroup and wave
    (4, 16, 128, 5000, "bf16"),      # 64 rows: four row tiles
    (3, 7, 96, 3001, "f16"),         # 21 rows: two row tiles, fp16
    (2, 1, 64, 300, "bf16"),         # anchor only
    (1, 4, 32, 1, "bf16"),           # one token, one step
    (5, 9, 1024, 40000, "f16"),
])
@pytest.mark.parametrize("packed", [False, True])
def test_lm_head_shapes(gpu_lib, B, K, hidden, V, dtype, packed):
    rng = np.random.default_rng(B * 1000 + K * 10 + hidden + V)
    li = W.make_lm_head(rng, B=B, K=K, hidden=hidden, V=V, dtype=dtype)
    say(f"[lm head] B={B} K={K} hidden={hidden} V={V} {dtype} packed={packed}")
    r_acc = _run(gpu_lib, li, packed)
    if V > 1:
        np.testing.assert_array_equal(r_acc, li.planted_len)


@pytest.mark.parametrize("packed", [False, True])
def test_lm_head_ties_take_the_lowest_index(gpu_lib, packed):
    """A vocabulary row duplicated later, and one duplicated earlier: equal logits from
    identical rows, so the lower index must win on both sides."""
    rng = np.random.default_rng(77)
    li = W.make_lm_head(rng, B=1, K=6, hidden=256, V=2000)
    w = li.weight.copy()
    t = li.planted_tok[0]
    w[1999] = w[t[0]]                 # later copy of row t0: t0 still wins
    w[0] = w[t[1]]                    # earlier copy of row t1: token 0 wins
    li2 = W.LmHeadInputs(1, 6, 256, 2000, "bf16", li.hidden_states, w, li.drafts,
                         li.planted_len, li.planted_tok)
    acc, toks, am = _call(gpu_lib, to_dev(li2.hidden_states, "bf16"), to_dev(li2.weight, "bf16"),
                          i32(li2.drafts), packed)
    torch.cuda.synchronize()
    r_acc, r_toks, r_am, _ = oracle.lm_head_greedy_ref(li2.hidden_states, w, li2.drafts, "bf16")
    np.testing.assert_array_equal(am.cpu().numpy(), r_am)
    assert r_am[0][0] == min(t[0], 1999) and r_am[0][1] == 0
    np.testing.assert_array_equal(toks.cpu().numpy(), r_toks)


# ------------------------------------------------------------------ un-steered inputs
def _bound(li, rows_idx, cols):
    """fp32 accumulation bound hidden * 2^-24 * sum_k |h_k w_vk| for the given entries."""
    h = np.abs(W.bf16_bits_to_f32(li.hidden_states).reshape(-1, li.hidden)).astype(np.float64)
    w = np.abs(W.bf16_bits_to_f32(li.weight[cols])).astype(np.float64)
    return li.hidden * 2.0 ** -24 * (h[rows_idx] * w).sum(axis=-1)


@pytest.mark.parametrize("B,K,hidden,V,packed", [(1, 16, 3584, 152064, False),
                                                 (1, 16, 3584, 152064, True),
                                                 (2, 8, 1024, 50000, False),
                                                 (2, 8, 1024, 50000, True),
                                                 (4, 16, 256, 7000, False),
                                                 (4, 16, 256, 7000, True)])
def test_lm_head_unsteered(gpu_lib, B, K, hidden, V, packed):
    """Natural logits: hidden states N(0, 1) against W ~ N(0, 0.02), nothing steered, so
    the top-2 gaps are whatever they are.  On every row whose float64 top-2 gap exceeds
    the sum of the two entries' fp32 accumulation bounds the argmax must match bit for
    bit; a row inside that bound is reported, and the GPU's choice must lie within the
    bound of the maximum.  Drafts follow the oracle's argmax for a Geometric(0.25)
    prefix; accept lengths and tokens must match on every sequence whose examined rows
    are all outside the bound."""
    rng = np.random.default_rng([hidden, V, B])
    li = W.make_lm_head(rng, B=B, K=K, hidden=hidden, V=V, margin=0.0)
    logits = oracle.lm_head_logits_ref(li.hidden_states, li.weight, "bf16")
    t = np.argmax(logits, axis=-1).astype(np.int32)
    L = np.minimum(rng.geometric(0.25, size=B) - 1, K - 1)
    drafts = rng.integers(0, V, size=(B, K - 1)).astype(np.int32)
    for b in range(B):
        drafts[b, :L[b]] = t[b, :L[b]]
        if L[b] < K - 1:
            drafts[b, L[b]] = (t[b, L[b]] + 1) % V
    say(f"[lm head] unsteered B={B} K={K} hidden={hidden} V={V} packed={packed}")
    acc, toks, am = _call(gpu_lib, to_dev(li.hidden_states, "bf16"), to_dev(li.weight, "bf16"),
                          i32(drafts), packed)
    torch.cuda.synchronize()
    acc, toks, am = acc.cpu().numpy(), toks.cpu().numpy(), am.cpu().numpy()
    r_acc, r_toks, r_am, _ = oracle.lm_head_greedy_ref(li.hidden_states, li.weight, drafts,
                                                       "bf16")
    flat = logits.reshape(B * K, V)
    order = np.argsort(-flat, axis=1, kind="stable")[:, :2]
    rows = np.arange(B * K)
    b1 = _bound(li, rows, order[:, 0])
    b2 = _bound(li, rows, order[:, 1])
    gap = flat[rows, order[:, 0]] - flat[rows, order[:, 1]]
    ambiguous = gap <= b1 + b2
    g = am.reshape(-1)
    bg = _bound(li, rows, g)
    assert (flat[rows, g] >= flat[rows, order[:, 0]] - (b1 + bg)).all()
    clear = ~ambiguous
    np.testing.assert_array_equal(g[clear], r_am.reshape(-1)[clear])
    amb = ambiguous.reshape(B, K)
    checked = 0
    for b in range(B):
        if not amb[b, :int(r_acc[b]) + 1].any():
            assert acc[b] == r_acc[b] and (toks[b] == r_toks[b]).all(), b
            checked += 1
    say(f"  smallest top-2 gap {gap.min():.3e} (bound there {(b1 + b2)[gap.argmin()]:.3e}); "
        f"rows inside the bound {int(ambiguous.sum())}/{B * K}, of which the GPU took another "
        f"token {int((g[ambiguous] != r_am.reshape(-1)[ambiguous]).sum())}; sequences "
        f"compared exactly {checked}/{B}")
