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


def _run(sv, li):
    acc, toks, am = sv.lm_head_greedy(to_dev(li.hidden_states, li.dtype),
                                      to_dev(li.weight, li.dtype), i32(li.drafts))
    torch.cuda.synchronize()
    r_acc, r_toks, r_am, _ = oracle.lm_head_greedy_ref(li.hidden_states, li.weight, li.drafts,
                                                       li.dtype)
    np.testing.assert_array_equal(am.cpu().numpy(), r_am)
    np.testing.assert_array_equal(acc.cpu().numpy(), r_acc)
    np.testing.assert_array_equal(toks.cpu().numpy(), r_toks)
    return r_acc


def test_qwen7b_lm_head_full_size(gpu_lib):
    li = W.make_workload_lm_head()
    say(f"[lm head] qwen7b_lmhead B={li.B} K={li.K} hidden={li.hidden} V={li.V}")
    r_acc = _run(gpu_lib, li)
    np.testing.assert_array_equal(r_acc, li.planted_len)


@pytest.mark.parametrize("B,K,hidden,V,dtype", [
    (1, 16, 512, 1000, "bf16"),
    (2, 8, 256, 777, "bf16"),        # ragged last workgroup and wave
    (4, 16, 128, 5000, "bf16"),      # 64 rows: four row tiles
    (3, 7, 96, 3001, "f16"),         # 21 rows: two row tiles, fp16
    (2, 1, 64, 300, "bf16"),         # anchor only
    (1, 4, 32, 1, "bf16"),           # one token, one step
    (5, 9, 1024, 40000, "f16"),
])
def test_lm_head_shapes(gpu_lib, B, K, hidden, V, dtype):
    rng = np.random.default_rng(B * 1000 + K * 10 + hidden + V)
    li = W.make_lm_head(rng, B=B, K=K, hidden=hidden, V=V, dtype=dtype)
    say(f"[lm head] B={B} K={K} hidden={hidden} V={V} {dtype}")
    r_acc = _run(gpu_lib, li)
    if V > 1:
        np.testing.assert_array_equal(r_acc, li.planted_len)


def test_lm_head_ties_take_the_lowest_index(gpu_lib):
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
    acc, toks, am = gpu_lib.lm_head_greedy(to_dev(li2.hidden_states, "bf16"),
                                           to_dev(li2.weight, "bf16"), i32(li2.drafts))
    torch.cuda.synchronize()
    r_acc, r_toks, r_am, _ = oracle.lm_head_greedy_ref(li2.hidden_states, w, li2.drafts, "bf16")
    np.testing.assert_array_equal(am.cpu().numpy(), r_am)
    assert r_am[0][0] == min(t[0], 1999) and r_am[0][1] == 0
    np.testing.assert_array_equal(toks.cpu().numpy(), r_toks)
