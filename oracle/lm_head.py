"""Reference LM head + greedy acceptance in float64 (test infrastructure).

The verify forward ends in the target's LM head; greedy acceptance takes the argmax of
each block row's logits over the vocabulary (VFlash-FM page, caption of the cycle
figure: the prefix matching the target's own greedy choice is accepted and the target
supplies the token at the first disagreement; the target is the unchanged model, so its
logits are hidden state . W_lm^T).  Here the logits are that product written out in
float64 from the stored (bf16) operands, and the acceptance is the chain rule.
"""
import numpy as np

from .accept import accept_greedy_ref
from .numerics import decode


def lm_head_logits_ref(hidden_states, weight, dtype: str, chunk: int = 1 << 14):
    """logits[b][i][v] = <hidden_states[b][i], weight[v]> in float64."""
    h = decode(hidden_states, dtype)
    B, K, H = h.shape
    V = weight.shape[0]
    hm = h.reshape(B * K, H)
    out = np.empty((B * K, V))
    for v0 in range(0, V, chunk):                  # vocabulary chunks bound the memory
        out[:, v0:v0 + chunk] = hm @ decode(weight[v0:v0 + chunk], dtype).T
    return out.reshape(B, K, V)


def lm_head_greedy_ref(hidden_states, weight, drafts, dtype: str):
    """Greedy acceptance over the LM head's logits.  Returns (accept_len, out_tokens,
    argmax) as accept_greedy_ref does, plus the float64 logits."""
    logits = lm_head_logits_ref(hidden_states, weight, dtype)
    acc, out, t = accept_greedy_ref(logits, drafts, "f32")      # float64 passes unchanged
    return acc, out, t, logits
