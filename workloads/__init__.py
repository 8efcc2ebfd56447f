"""Seeded synthetic inputs for block verification, shared by the tests and the bench.

This module only draws random inputs and lays them out; it performs none of the
verification arithmetic (no attention, no argmax of target rows, no softmax, no
acceptance test).  Both the float64 oracle and the GPU library consume what it
produces, and neither imports the other.

Workloads (shapes taken from the pages' measurement setups):

* ``tiny_fp32``      -- 1 layer, 2 query heads on 1 KV head, head_dim 64, context
  512, block 4 (anchor + 3 drafts), fp32 Q/K/V ~ N(0,1), vocabulary 1000,
  fp32 logits ~ N(0,3), greedy acceptance.
* ``qwen7b_25k``     -- 7B-shaped verify layer (28 q heads, 4 KV heads, d 128),
  bf16 KV cache of 25,119 context tokens plus the 16 block tokens, block 16 with
  the in-block causal mask, bf16 logits [16 x 152,064] ~ N(0,3), greedy.  The
  context length is the one of the VFlash-FM demo cycle (VFlash-FM page, "How
  VFlash-FM works", cycle figure), block 16 from its demo setup.
* ``batched_paged``  -- 8 sequences, contexts log-uniform in [4096, 32768),
  paged bf16 KV with 16-token pages and one globally shuffled page pool.
* ``compressor_sar`` -- SpecFLASH latent compressor (SpecFLASH README,
  "components", compressor equation): 32 images, D = 4096, (C, N) = (64, 576)
  and (36, 324), fp16 queries ~ N(0, 0.02), features ~ N(0, 1); followed by
  the semi-autoregressive block of 5 slot queries, 64 heads x 64.
* ``qwen72b_sampling`` -- 72B-shaped sampling verify (64 q heads, 8 KV heads,
  d 128), bf16 KV of 25,000 context tokens, block 32, target logits ~ N(0,3),
  draft logits = bf16(target + N(0,1)), temperature 1.
* ``qwen7b_tree60`` -- the 7B layer verifying a static draft tree of 60 nodes
  below the anchor (the "Tree-60" variant of the VFlash-FM results table): 61
  block rows with ancestor masks, planted greedy path through the tree.
* ``vflash_drafter`` -- one layer of the VFlash-FM drafter's block attention: the
  anchor and 15 masks attend bidirectionally to each other and to keys/values over
  the whole 25,119-token context (VFlash-FM page, cycle figure: 4 drafter layers
  reading projected keys and values of the target's cached hidden states), in the
  7B layer's head geometry.
* ``qwen7b_lmhead`` -- the 7B target's LM head over the block: 16 hidden states of
  width 3584 against a 152,064 x 3584 bf16 output embedding ~ N(0, 0.02), each
  hidden state steered to a planted token, drafts with a planted prefix.

Conventions (fixed here, used by both sides):

* "N(mu, s)" takes s as the standard deviation.
* bf16 tensors are carried as ``uint16`` bit patterns, rounded from float32
  draws with round-to-nearest-even.
* KV caches are paged.  K pages are ``[num_pages][Hkv][P][d]`` (token-major);
  V pages are ``[num_pages][Hkv][d][P]`` (dim-major).  ``page_table[b][j]``
  is the physical page holding tokens ``[j*P, (j+1)*P)`` of sequence b.  The
  cache of sequence b holds ``ctx_lens[b] + K`` tokens: the context followed
  by the block's own K/V rows.
* Planted greedy prefix: every target row gets one planted maximum (value 20,
  all other entries are clipped to +-19.5 = 6.5 sigma), so the lowest-index
  argmax of each row is known by construction.  A quarter of the rows repeat
  the maximum at a later index, which exercises the lowest-index tie rule.
  Drafts copy the planted maxima for a Geometric(0.25) prefix length L
  (P(L = k) = 0.75^k * 0.25, truncated to K-1); the next draft is drawn
  uniformly from the other tokens and later drafts uniformly from all tokens,
  so the accepted length equals L by construction.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "WORKLOADS", "bf16_bits", "bf16_bits_to_f32", "VerifyInputs", "GreedyInputs",
    "SampleInputs", "CompressInputs", "SarInputs", "make_verify", "make_greedy",
    "make_sample", "make_compress", "make_sar", "build_page_table", "causal_mask",
    "all_ones_mask", "rng_for", "TreeInputs", "TREE60_LEVELS", "make_tree_topology",
    "chain_topology", "tree_mask", "make_tree_greedy", "workload_tree",
    "make_workload_tree", "LmHeadInputs", "make_lm_head", "make_workload_lm_head",
    "TreeSampleInputs", "make_tree_sample", "make_workload_tree_sample",
]

BASE_SEED = 1000
PLANT_VALUE = 20.0       # planted row maximum (exact in bf16 and fp32)
PLANT_CLIP = 19.5        # every other logit is clipped to [-19.5, 19.5]
TIE_FRACTION = 0.25      # rows that repeat the planted maximum at a later index


# --------------------------------------------------------------------------- dtypes

def bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if u.size and int(u.max()) >= 0xFFFF8000:   # negative NaN payloads: widen to 64 bits
        w = u.astype(np.uint64)
        return ((w + 0x7FFF + ((w >> 16) & 1)) >> 16).astype(np.uint16)
    r = (u >> 16) & 1                           # round half to even, in place
    r += 0x7FFF
    r += u
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits(x)
    if dtype == "f16":
        return np.ascontiguousarray(x, dtype=np.float16)
    raise ValueError(dtype)


def _normal(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return _round_to(x, dtype)


def rng_for(workload: str, cycle: int = 0) -> np.random.Generator:
    """The generator for a workload's cycle: SeedSequence([1000 + index, cycle])."""
    idx = list(WORKLOADS).index(workload) + 1
    return np.random.default_rng(np.random.SeedSequence([BASE_SEED + idx, cycle]))


# --------------------------------------------------------------------------- masks

def causal_mask(K: int) -> np.ndarray:
    """Row i sees block keys 0..i (bit t of row i set iff t <= i)."""
    return np.array([(1 << (i + 1)) - 1 for i in range(K)], dtype=np.uint64)


def all_ones_mask(K: int) -> np.ndarray:
    """Every row sees every block key (one bidirectional block)."""
    full = (1 << K) - 1
    return np.array([full] * K, dtype=np.uint64)


# --------------------------------------------------------------------------- paging

def build_page_table(rng: Optional[np.random.Generator], n_tokens: np.ndarray, P: int,
                     shuffle: bool):
    """Assign physical pages to sequences.

    Returns (page_table int32 [B][max_pages], num_pages).  Pages are drawn from
    one pool; with ``shuffle`` a random permutation scatters them across all
    sequences, otherwise sequence b owns a contiguous run (identity table for
    B = 1).  Unused table entries are -1.
    """
    n_tokens = np.asarray(n_tokens, dtype=np.int64)
    pages_per = (n_tokens + P - 1) // P
    num_pages = int(pages_per.sum())
    pool = np.arange(num_pages, dtype=np.int32)
    if shuffle:
        pool = rng.permutation(num_pages).astype(np.int32)
    max_pages = int(pages_per.max())
    table = np.full((len(n_tokens), max_pages), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages_per):
        table[b, :n] = pool[off:off + n]
        off += n
    return table, num_pages


# --------------------------------------------------------------------------- verify

@dataclass
class VerifyInputs:
    """Inputs of one verify-attention call (one layer)."""
    B: int
    K: int
    Hq: int
    Hkv: int
    D: int
    P: int
    dtype: str                      # "f32" | "bf16" | "f16"
    q: np.ndarray                   # [B][K][Hq][D]
    k_cache: np.ndarray             # [num_pages][Hkv][P][D]
    v_cache: np.ndarray             # [num_pages][Hkv][D][P]
    page_table: np.ndarray          # int32 [B][max_pages]
    ctx_lens: np.ndarray            # int32 [B] (tokens before the block)
    mask: np.ndarray                # uint64 [K] row bitmasks over block keys
    scale: float = 0.0              # 0 -> 1/sqrt(D)

    @property
    def num_pages(self) -> int:
        return self.k_cache.shape[0]

    @property
    def n_keys(self) -> np.ndarray:
        return self.ctx_lens.astype(np.int64) + self.K

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes: every visible (context + block) key and value, once."""
        esz = 4 if self.dtype == "f32" else 2
        return int(self.n_keys.sum()) * self.Hkv * self.D * 2 * esz


def make_verify(rng: np.random.Generator, *, B: int, K: int, Hq: int, Hkv: int, D: int,
                ctx_lens, P: int = 16, dtype: str = "bf16", shuffle: bool = False,
                mask: Optional[np.ndarray] = None, qk_std: float = 1.0) -> VerifyInputs:
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32).reshape(B)
    n_tokens = ctx_lens.astype(np.int64) + K
    page_table, num_pages = build_page_table(rng, n_tokens, P, shuffle)
    q = _normal(rng, (B, K, Hq, D), qk_std, dtype)
    k_cache = _normal(rng, (num_pages, Hkv, P, D), qk_std, dtype)
    v_cache = _normal(rng, (num_pages, Hkv, D, P), 1.0, dtype)
    if mask is None:
        mask = causal_mask(K)
    return VerifyInputs(B, K, Hq, Hkv, D, P, dtype, q, k_cache, v_cache, page_table,
                        ctx_lens, np.asarray(mask, dtype=np.uint64))


def log_uniform_contexts(rng: np.random.Generator, B: int, lo: int = 4096,
                         hi: int = 32768) -> np.ndarray:
    """ctx = floor(exp(U(ln lo, ln hi)))."""
    u = rng.uniform(np.log(lo), np.log(hi), size=B)
    return np.floor(np.exp(u)).astype(np.int32)


# --------------------------------------------------------------------------- greedy

@dataclass
class GreedyInputs:
    B: int
    K: int
    V: int
    dtype: str                 # "f32" | "bf16"
    logits: np.ndarray         # [B][K][V]
    drafts: np.ndarray         # int32 [B][K-1]; drafts[b][k-1] is draft d_k
    planted_len: np.ndarray    # int32 [B]: accepted length by construction
    planted_tok: np.ndarray    # int32 [B][K]: lowest-index maximum of each row


def _planted_logits(rng: np.random.Generator, B: int, K: int, V: int, dtype: str,
                    std: float):
    """Target logits [B][K][V] with one planted maximum per row (and planted ties)."""
    x = rng.standard_normal(size=(B, K, V), dtype=np.float32)
    x *= np.float32(std)
    np.clip(x, -PLANT_CLIP, PLANT_CLIP, out=x)
    tok = rng.integers(0, V, size=(B, K)).astype(np.int32)
    tie = rng.random(size=(B, K)) < TIE_FRACTION
    tie_u = rng.random(size=(B, K))
    bb, kk = np.meshgrid(np.arange(B), np.arange(K), indexing="ij")
    x[bb, kk, tok] = PLANT_VALUE
    for b in range(B):
        for k in range(K):
            t = int(tok[b, k])
            if tie[b, k] and t < V - 1:
                j = t + 1 + int(tie_u[b, k] * (V - 1 - t))
                x[b, k, min(j, V - 1)] = PLANT_VALUE
    return _round_to(x, dtype), tok


def make_greedy(rng: np.random.Generator, *, B: int, K: int, V: int, dtype: str = "bf16",
                std: float = 3.0) -> GreedyInputs:
    logits, tok = _planted_logits(rng, B, K, V, dtype, std)
    L = np.minimum(rng.geometric(0.25, size=B) - 1, K - 1).astype(np.int32)
    drafts = rng.integers(0, V, size=(B, K - 1)).astype(np.int32)
    other = rng.integers(0, max(V - 1, 1), size=B).astype(np.int32)
    if V == 1:                      # one token: every draft is the argmax
        L[:] = K - 1
    for b in range(B):
        n = int(L[b])
        drafts[b, :n] = tok[b, :n]
        if n < K - 1:
            t = int(tok[b, n])
            o = int(other[b])
            drafts[b, n] = o if o < t else o + 1
    return GreedyInputs(B, K, V, dtype, logits, drafts, L, tok)


# --------------------------------------------------------------------------- trees

# Tree-60: 60 draft nodes below the anchor, by depth (a static draft tree of the kind
# the VFlash-FM results table verifies as "Tree-60"; the level sizes are this module's
# choice, the pages give only the node count).
TREE60_LEVELS = (10, 20, 16, 8, 4, 2)


def make_tree_topology(rng: np.random.Generator, levels=TREE60_LEVELS) -> np.ndarray:
    """Parents int32 [n] of draft nodes 1..n (node 0 is the anchor).

    Nodes are numbered level by level; each node of a level hangs under a uniformly
    drawn node of the better-ranked half of the previous level (the anchor for level
    1), so a parent always has a smaller number than its children.
    """
    parents = []
    prev = [0]
    nid = 1
    for size in levels:
        top = prev[:max(1, (len(prev) + 1) // 2)]
        cur = []
        for _ in range(size):
            parents.append(top[int(rng.integers(0, len(top)))])
            cur.append(nid)
            nid += 1
        prev = cur
    return np.asarray(parents, dtype=np.int32)


def chain_topology(n: int) -> np.ndarray:
    """The chain as a tree: node i hangs under node i-1."""
    return np.arange(n, dtype=np.int32)


def tree_mask(parents) -> np.ndarray:
    """Block-mask rows of a tree: row i sees node i and every ancestor of it."""
    parents = np.asarray(parents)
    K = len(parents) + 1
    rows = [1]
    for i in range(1, K):
        rows.append((1 << i) | rows[int(parents[i - 1])])
    return np.array(rows, dtype=np.uint64)


@dataclass
class TreeInputs:
    B: int
    K: int                     # nodes, anchor included
    V: int
    dtype: str
    logits: np.ndarray         # [B][K][V]: target row of every node
    parents: np.ndarray        # int32 [B][K-1]: parent of node i at [b][i-1]
    tokens: np.ndarray         # int32 [B][K-1]: draft token of node i at [b][i-1]
    planted_len: np.ndarray    # int32 [B]: accepted depth by construction
    planted_path: np.ndarray   # int32 [B][K]: anchor, accepted nodes, then -1
    planted_tok: np.ndarray    # int32 [B][K]: lowest-index maximum of each row


def make_tree_greedy(rng: np.random.Generator, *, B: int, V: int, parents,
                     dtype: str = "bf16", std: float = 3.0) -> TreeInputs:
    """Planted target rows over a draft tree with a planted accepted path.

    Siblings carry distinct tokens.  A Geometric(0.25) depth L is drawn per sequence;
    from the anchor, L times (while the node has children) a uniformly drawn child
    takes the planted maximum of its parent's row (trading tokens with the sibling
    that held it), and finally no child of the last node keeps that node's maximum.
    """
    parents = np.asarray(parents, dtype=np.int32)
    K = len(parents) + 1
    logits, tok = _planted_logits(rng, B, K, V, dtype, std)
    children = [[] for _ in range(K)]
    for i in range(1, K):
        children[int(parents[i - 1])].append(i)
    tokens = np.zeros((B, K), dtype=np.int64)
    for b in range(B):
        for u in range(K):
            if children[u]:
                tokens[b, children[u]] = rng.choice(V, size=len(children[u]), replace=False)
    L = rng.geometric(0.25, size=B) - 1
    plen = np.zeros(B, dtype=np.int32)
    path = np.full((B, K), -1, dtype=np.int32)
    for b in range(B):
        cur, depth = 0, 0
        path[b, 0] = 0
        while depth < L[b] and children[cur]:
            ch = children[cur]
            c = ch[int(rng.integers(0, len(ch)))]
            want = int(tok[b, cur])
            for sib in ch:
                if tokens[b, sib] == want:
                    tokens[b, sib] = tokens[b, c]
            tokens[b, c] = want
            cur = c
            depth += 1
            path[b, depth] = c
        want = int(tok[b, cur])
        taken = {int(tokens[b, s]) for s in children[cur]}
        for s in children[cur]:
            if tokens[b, s] == want:
                t = int(rng.integers(0, V))
                while t == want or t in taken:
                    t = int(rng.integers(0, V))
                tokens[b, s] = t
                taken.add(t)
        plen[b] = depth
    return TreeInputs(B, K, V, dtype, logits, np.tile(parents, (B, 1)),
                      tokens[:, 1:].astype(np.int32), plen, path, tok)


# --------------------------------------------------------------------------- LM head

@dataclass
class LmHeadInputs:
    B: int
    K: int
    hidden: int
    V: int
    dtype: str                 # "bf16"
    hidden_states: np.ndarray  # [B][K][hidden]: the verify pass's last hidden states
    weight: np.ndarray         # [V][hidden]: the LM head (output embedding)
    drafts: np.ndarray         # int32 [B][K-1]
    planted_len: np.ndarray    # int32 [B]
    planted_tok: np.ndarray    # int32 [B][K]: the token each row is steered to


def make_lm_head(rng: np.random.Generator, *, B: int, K: int, hidden: int, V: int,
                 dtype: str = "bf16", w_std: float = 0.02, margin: float = 20.0,
                 chunk: int = 1 << 14) -> LmHeadInputs:
    """Random LM head W ~ N(0, w_std) [V][hidden]; hidden state of row i =
    s * W[t_i] + N(0, 1) with s = margin / (hidden * w_std^2), which puts the planted
    token t_i's logit near `margin` while the others stay within a few units of 0; drafts
    follow the planted tokens for a Geometric(0.25) prefix, as for planted logits."""
    steer = margin / (hidden * w_std * w_std)
    w = np.empty((V, hidden), dtype=np.uint16 if dtype == "bf16" else np.float32)
    for v0 in range(0, V, chunk):                  # drawn in row chunks, in order
        v1 = min(V, v0 + chunk)
        part = rng.standard_normal(size=(v1 - v0, hidden), dtype=np.float32)
        part *= np.float32(w_std)
        w[v0:v1] = _round_to(part, dtype)
    tok = rng.integers(0, V, size=(B, K)).astype(np.int32)
    wf = bf16_bits_to_f32(w[tok.reshape(-1)]) if dtype == "bf16" else w[tok.reshape(-1)]
    h = rng.standard_normal(size=(B * K, hidden), dtype=np.float32)
    h += np.float32(steer) * wf
    hs = _round_to(h.reshape(B, K, hidden), dtype)
    L = np.minimum(rng.geometric(0.25, size=B) - 1, K - 1).astype(np.int32)
    drafts = rng.integers(0, V, size=(B, K - 1)).astype(np.int32)
    other = rng.integers(0, max(V - 1, 1), size=B).astype(np.int32)
    for b in range(B):
        n = int(L[b])
        drafts[b, :n] = tok[b, :n]
        if n < K - 1:
            t = int(tok[b, n])
            o = int(other[b])
            drafts[b, n] = o if o < t else o + 1
    return LmHeadInputs(B, K, hidden, V, dtype, hs, w, drafts, L, tok)


# --------------------------------------------------------------------------- sampling

@dataclass
class SampleInputs:
    B: int
    K: int
    V: int
    dtype: str                 # "f32" | "bf16"
    target_logits: np.ndarray  # [B][K][V]
    draft_logits: np.ndarray   # [B][K-1][V]; row k-1 is the draft distribution of d_k
    drafts: np.ndarray         # int32 [B][K-1]
    temperature: float
    seed: int
    offset: int


def _to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def make_sample(rng: np.random.Generator, *, B: int, K: int, V: int, dtype: str = "bf16",
                temperature: float = 1.0, std: float = 3.0, noise: float = 1.0,
                seed: int = 0x5EED, offset: int = 0) -> SampleInputs:
    """Target logits ~ N(0, std); draft logits = round(target + N(0, noise)).

    The drafts are drawn from the draft distribution softmax(draft/T) with the
    Gumbel-max trick; this plays the drafter's part and is not verification.
    """
    tl = rng.standard_normal(size=(B, K, V), dtype=np.float32)
    tl *= np.float32(std)
    target = _round_to(tl, dtype)
    t32 = _to_f64(target, dtype).astype(np.float32)
    dn = rng.standard_normal(size=(B, K - 1, V), dtype=np.float32)
    dn *= np.float32(noise)
    draft = _round_to(t32[:, :K - 1, :] + dn, dtype)
    g = -np.log(-np.log(rng.random(size=(B, K - 1, V))))
    drafts = np.argmax(_to_f64(draft, dtype) / temperature + g, axis=-1).astype(np.int32)
    return SampleInputs(B, K, V, dtype, target, draft, drafts, float(temperature),
                        int(seed), int(offset))


@dataclass
class TreeSampleInputs:
    B: int
    K: int                     # nodes, anchor included
    V: int
    dtype: str
    target_logits: np.ndarray  # [B][K][V]: target row of every node
    draft_logits: np.ndarray   # [B][K-1][V]: row i-1 = the distribution node i was drawn from
    parents: np.ndarray        # int32 [K-1]: the tree (shared by the batch)
    tokens: np.ndarray         # int32 [B][K-1]
    temperature: float
    seed: int
    offset: int


def make_tree_sample(rng: np.random.Generator, *, B: int, V: int, parents, dtype: str = "bf16",
                     temperature: float = 1.0, std: float = 3.0, noise: float = 1.0,
                     seed: int = 0x5EED, offset: int = 0) -> TreeSampleInputs:
    """Target logits ~ N(0, std) for every node; the children of node u share one draft
    row, round(target row u + N(0, noise)), and draw their tokens from it independently
    (with replacement) by the Gumbel-max trick -- the drafter's part, not verification."""
    parents = np.asarray(parents, dtype=np.int32)
    K = len(parents) + 1
    tl = rng.standard_normal(size=(B, K, V), dtype=np.float32)
    tl *= np.float32(std)
    target = _round_to(tl, dtype)
    t32 = _to_f64(target, dtype).astype(np.float32)
    draft = np.empty((B, K - 1, V), dtype=target.dtype)
    tokens = np.zeros((B, K - 1), dtype=np.int32)
    for u in sorted(set(int(x) for x in parents)):
        kids = [i for i in range(1, K) if int(parents[i - 1]) == u]
        dn = rng.standard_normal(size=(B, V), dtype=np.float32)
        dn *= np.float32(noise)
        row = _round_to(t32[:, u, :] + dn, dtype)
        q64 = _to_f64(row, dtype) / temperature
        for i in kids:
            draft[:, i - 1, :] = row
            g = -np.log(-np.log(rng.random(size=(B, V))))
            tokens[:, i - 1] = np.argmax(q64 + g, axis=-1)
    return TreeSampleInputs(B, K, V, dtype, target, draft, parents, tokens, float(temperature),
                            int(seed), int(offset))


def make_workload_tree_sample(name: str = "qwen7b_tree60", cycle: int = 0,
                              B: int = 1) -> TreeSampleInputs:
    """Sampling verification of the static Tree-60 of the tree workload (T = 1)."""
    p = WORKLOADS[name].params
    return make_tree_sample(rng_for(name, 30_000 + cycle), B=B, V=p["V"],
                            parents=workload_tree(name), dtype=p["dtype"], offset=cycle)


# --------------------------------------------------------------------------- compressor

@dataclass
class CompressInputs:
    B: int
    C: int
    N: int
    D: int
    queries: np.ndarray   # float16 [C][D]
    feats: np.ndarray     # float16 [B][N][D]


def make_compress(rng: np.random.Generator, *, B: int, C: int, N: int, D: int,
                  q_std: float = 0.02, f_std: float = 1.0) -> CompressInputs:
    queries = _normal(rng, (C, D), q_std, "f16")
    feats = _normal(rng, (B, N, D), f_std, "f16")
    return CompressInputs(B, C, N, D, queries, feats)


@dataclass
class SarInputs:
    """Semi-autoregressive block: S slot queries over C context rows + S slot rows."""
    B: int
    S: int
    H: int
    D: int
    q: np.ndarray         # float16 [B][S][H][D]
    slot_k: np.ndarray    # float16 [B][S][H][D]
    slot_v: np.ndarray    # float16 [B][S][H][D]


def make_sar(rng: np.random.Generator, *, B: int, S: int = 5, H: int = 64,
             D: int = 64) -> SarInputs:
    return SarInputs(B, S, H, D, _normal(rng, (B, S, H, D), 1.0, "f16"),
                     _normal(rng, (B, S, H, D), 1.0, "f16"),
                     _normal(rng, (B, S, H, D), 1.0, "f16"))


# --------------------------------------------------------------------------- registry

@dataclass
class Workload:
    name: str
    desc: str
    params: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", "1 layer, 2q/1kv, d64, ctx 512, block 4, fp32, V 1000",
                          dict(B=1, K=4, Hq=2, Hkv=1, D=64, ctx=512, V=1000, dtype="f32")),
    "qwen7b_25k": Workload("qwen7b_25k", "28q/4kv d128 bf16, ctx 25119 + block 16, V 152064",
                           dict(B=1, K=16, Hq=28, Hkv=4, D=128, ctx=25119, V=152064,
                                dtype="bf16")),
    "batched_paged": Workload("batched_paged", "8 seqs, ctx log-uniform 4k-32k, shuffled pages",
                              dict(B=8, K=16, Hq=28, Hkv=4, D=128, V=152064, dtype="bf16")),
    "compressor_sar": Workload("compressor_sar", "B 32, D 4096, (64,576) and (36,324); SAR 5 slots",
                               dict(B=32, D=4096, shapes=((64, 576), (36, 324)), S=5, H=64,
                                    HD=64)),
    "qwen72b_sampling": Workload("qwen72b_sampling", "64q/8kv d128 bf16, ctx 25000 + block 32",
                                 dict(B=1, K=32, Hq=64, Hkv=8, D=128, ctx=25000, V=152064,
                                      dtype="bf16", T=1.0)),
    "qwen7b_tree60": Workload("qwen7b_tree60", "7B layer, ctx 25119 + Tree-60 (61 nodes), V 152064",
                              dict(B=1, K=61, Hq=28, Hkv=4, D=128, ctx=25119, V=152064,
                                   dtype="bf16", levels=TREE60_LEVELS)),
    "qwen7b_lmhead": Workload("qwen7b_lmhead", "7B LM head: 16 rows x hidden 3584 x V 152064",
                              dict(B=1, K=16, hidden=3584, V=152064, dtype="bf16")),
    "vflash_drafter": Workload("vflash_drafter", "drafter layer: anchor + 15 masks, bidirectional "
                               "block over ctx 25119, 28q/4kv d128",
                               dict(B=1, K=16, Hq=28, Hkv=4, D=128, ctx=25119, dtype="bf16")),
}


def workload_tree(name: str) -> np.ndarray:
    """The static draft tree of a tree workload (parents of nodes 1..K-1)."""
    return make_tree_topology(rng_for(name, 20_000), WORKLOADS[name].params["levels"])


def make_workload_verify(name: str, cycle: int = 0) -> VerifyInputs:
    """Verify-attention inputs of a named workload (draw order: contexts, pages, Q, K, V)."""
    p = WORKLOADS[name].params
    rng = rng_for(name, cycle)
    if name == "qwen7b_tree60":
        return make_verify(rng, B=p["B"], K=p["K"], Hq=p["Hq"], Hkv=p["Hkv"], D=p["D"],
                           ctx_lens=[p["ctx"]] * p["B"], P=16, dtype=p["dtype"],
                           mask=tree_mask(workload_tree(name)))
    if name == "vflash_drafter":
        return make_verify(rng, B=p["B"], K=p["K"], Hq=p["Hq"], Hkv=p["Hkv"], D=p["D"],
                           ctx_lens=[p["ctx"]] * p["B"], P=16, dtype=p["dtype"],
                           mask=all_ones_mask(p["K"]))
    if name == "batched_paged":
        ctx = log_uniform_contexts(rng, p["B"])
        return make_verify(rng, B=p["B"], K=p["K"], Hq=p["Hq"], Hkv=p["Hkv"], D=p["D"],
                           ctx_lens=ctx, P=16, dtype=p["dtype"], shuffle=True)
    return make_verify(rng, B=p["B"], K=p["K"], Hq=p["Hq"], Hkv=p["Hkv"], D=p["D"],
                       ctx_lens=[p["ctx"]] * p["B"], P=16, dtype=p["dtype"])


def make_workload_greedy(name: str, cycle: int = 0) -> GreedyInputs:
    p = WORKLOADS[name].params
    rng = rng_for(name, 10_000 + cycle)
    return make_greedy(rng, B=p["B"], K=p["K"], V=p["V"], dtype=p["dtype"])


def make_workload_sample(name: str, cycle: int = 0) -> SampleInputs:
    p = WORKLOADS[name].params
    rng = rng_for(name, 10_000 + cycle)
    return make_sample(rng, B=p["B"], K=p["K"], V=p["V"], dtype=p["dtype"],
                       temperature=p["T"], seed=0x5EED, offset=cycle)


def make_workload_tree(name: str, cycle: int = 0) -> TreeInputs:
    p = WORKLOADS[name].params
    rng = rng_for(name, 10_000 + cycle)
    return make_tree_greedy(rng, B=p["B"], V=p["V"], parents=workload_tree(name),
                            dtype=p["dtype"])


def make_workload_lm_head(name: str = "qwen7b_lmhead", cycle: int = 0) -> LmHeadInputs:
    p = WORKLOADS[name].params
    return make_lm_head(rng_for(name, cycle), B=p["B"], K=p["K"], hidden=p["hidden"], V=p["V"],
                        dtype=p["dtype"])
