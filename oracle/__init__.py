"""Float64 CPU oracle for block verification -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct restatement of what the
verification hot path computes.  Only the test suite, the smoke check and the
bench's CPU-baseline leg may import it; the library and its Python binding
never do, and it shares no code with them.

Every function follows a passage of the pages it cites:

* ``attention.verify_attention_ref`` -- the target scores every block position
  in one forward over the whole context plus the block (VFlash-FM page, "How
  VFlash-FM works" and the cycle figure), with native grouped-query attention
  (VFlash-FM page, demo setup).
* ``accept.accept_greedy_ref`` -- the prefix that matches the target's greedy
  choice is accepted and the target supplies the token at the first
  disagreement (VFlash-FM page, caption of the cycle figure).
* ``accept.sample_rule`` / ``accept.accept_sample_ref`` -- the standard
  speculative acceptance-rejection rule (SpecFLASH README, "components",
  verification paragraph; the speculative-sampling references listed on the
  SpecFLASH mlsanity page).
* ``philox.philox4x64_10`` -- counter-based Philox4x64-10 (Salmon et al.,
  SC'11), the uniform source of the sampling rule.
* ``compress.latent_compress_ref`` -- softmax(C . F_V^T) . F_V (SpecFLASH
  README, "components", compressor equation).
* ``kv.kv_append_ref`` -- writing the block's rows into the preallocated paged
  KV cache (VFlash-FM page, demo setup).
* ``kv.commit_ref`` -- closing a cycle: the context grows by the accepted drafts
  plus the anchor, and the target's correction becomes the next anchor (VFlash-FM
  page, caption of the cycle figure).
* ``tree.accept_greedy_tree_ref`` / ``tree.tree_commit_ref`` -- greedy verification
  of a draft tree (the "Tree-60" row of the VFlash-FM results table) read as the
  chain rule walked from the anchor, and the commit that moves the accepted path's
  K/V rows into place.
* ``tree_sample.accept_sample_tree_ref`` / ``tree_sample.sample_tree_rule`` -- sampling
  verification of a draft tree (the "Tree-60" row of the VFlash-FM results table with the
  standard acceptance-rejection rule of the SpecFLASH README): recursive rejection over
  the children of the current node, which reduces to the chain rule on a chain.
* ``lm_head.lm_head_greedy_ref`` -- the target's LM head (hidden state . W^T) followed
  by greedy acceptance over its logits (VFlash-FM page, caption of the cycle figure).

Parity pins: every function is pinned in ``tests/test_oracle_*.py`` against
something other than itself (worked example, library routine, closed form,
invariant or exhaustive enumeration).  No function here is "parity unpinned".
"""
from .numerics import decode
from .attention import verify_attention_ref, single_query_ref, merge_partials_ref
from .accept import accept_greedy_ref, sample_rule, accept_sample_ref, race_ref
from .philox import philox4x64_10, uniforms, ACCEPT, RESAMPLE
from .compress import latent_compress_ref
from .kv import kv_append_ref, commit_ref
from .tree import accept_greedy_tree_ref, tree_commit_ref
from .lm_head import lm_head_logits_ref, lm_head_greedy_ref
from .tree_sample import accept_sample_tree_ref, sample_tree_rule, children_of

__all__ = [
    "decode", "verify_attention_ref", "single_query_ref", "merge_partials_ref",
    "accept_greedy_ref", "sample_rule", "accept_sample_ref", "race_ref",
    "philox4x64_10", "uniforms", "ACCEPT", "RESAMPLE", "latent_compress_ref",
    "kv_append_ref", "commit_ref", "accept_greedy_tree_ref", "tree_commit_ref",
    "lm_head_logits_ref", "lm_head_greedy_ref", "accept_sample_tree_ref", "sample_tree_rule",
    "children_of",
]
