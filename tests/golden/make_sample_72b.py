"""Writes tests/golden/sample_72b_1024.json: the float64 oracle's sampling verdicts on
1,024 sequence-cycles of the 72B sampling shape (8 sequences, K = 32, vocabulary 152,064,
temperature 1, Philox seed 0x5EED, offsets 0 .. 127).

Only the seeded input generators (workloads/) and the oracle (oracle/) are called; no
value here comes from the GPU library.  The GPU parity test regenerates the same inputs,
checks their digest against the one stored here, and compares the library's outputs
with these verdicts.

    python tests/golden/make_sample_72b.py        # ~5 CPU-minutes, uses every core
"""
import hashlib
import json
import os
import sys
from concurrent.futures import ProcessPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads as W  # noqa: E402

OUT = os.path.join(HERE, "sample_72b_1024.json")
OFFSETS = 128


def inputs():
    """The eight sequences every offset verifies (drawn once from the workload's seed)."""
    p = W.WORKLOADS["qwen72b_sampling"].params
    return W.make_sample(W.rng_for("qwen72b_sampling", 50_000), B=8, K=p["K"], V=p["V"],
                         dtype=p["dtype"], temperature=p["T"], seed=0x5EED, offset=0)


def digest(s) -> str:
    h = hashlib.sha256()
    for a in (s.target_logits, s.draft_logits, s.drafts):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()[:16]


def _one(off):
    s = inputs()
    acc, out, diag = oracle.accept_sample_ref(s.target_logits, s.draft_logits, s.drafts,
                                              s.dtype, s.temperature, s.seed, off,
                                              return_diag=True)
    return off, [int(a) for a in acc], [int(out[b, acc[b]]) for b in range(s.B)], \
        [_short(d[0]) for d in diag], [_short(d[1]) for d in diag]


def _short(x):
    """A diagnostic to 4 significant digits (reported, never compared)."""
    return float(f"{float(x):.3e}")


def main():
    s = inputs()
    rows = {}
    with ProcessPoolExecutor(max_workers=max(1, len(os.sched_getaffinity(0)) // 2)) as ex:
        for off, acc, tok, margin, gap in ex.map(_one, range(OFFSETS)):
            rows[off] = {"accept_len": acc, "token": tok, "margin": margin, "race_gap": gap}
    doc = {
        "what": "oracle.accept_sample_ref verdicts: accept_len[b] and the drawn token "
                "out_tokens[b][accept_len[b]] (the accepted drafts before it are the "
                "inputs' own), with the smallest |u - threshold| and race gap per sequence",
        "workload": "qwen72b_sampling shape: B 8, K 32, V 152064, bf16 logits, T 1",
        "generator": "workloads.make_sample(rng_for('qwen72b_sampling', 50000), ...)",
        "seed": 0x5EED,
        "input_digest": digest(s),
        "offsets": {str(k): rows[k] for k in sorted(rows)},
    }
    with open(OUT, "w") as fh:
        json.dump(doc, fh, separators=(",", ":"))
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
