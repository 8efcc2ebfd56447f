"""Verify-cycle benchmark on one MI355X.

One step = one verify cycle of the 7B-shaped workload (28 q heads / 4 KV heads, d 128,
bf16 KV cache of 25,119 context tokens + the 16 block tokens, block 16):
sv_verify_attention (split-KV pass + merge pass) followed by sv_accept_greedy on the
[16 x 152,064] bf16 logits.  Inputs are seeded synthetic data, resident in HBM before
timing; the KV caches and logits rotate over copies whose total exceeds twice the
256 MB last-level cache, so every cycle streams its KV from HBM.

Prints one JSON line.  Extra fields: the attention pass's live-measured duration and
KV-read bandwidth, its roofline against 8 TB/s, and the float64 CPU oracle's rate on
a bounded sample of the same workload.
"""
import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
COPY_BYTES = 256 << 20           # calibration copy: bytes read and written per launch
WORKLOAD = "qwen7b_25k"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--copies", type=int, default=12, help="rotated KV/logit copies")
    ap.add_argument("--split-keys", type=int, default=0)
    ap.add_argument("--launch", choices=["graph", "direct"], default="graph")
    ap.add_argument("--attn-reps", type=int, default=1000,
                    help="attention-only launches timed for the roofline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--pmc-workload", choices=["attn", "copy"], default=None,
                    help="run a fixed loop for rocprofv3 --pmc counter passes and exit: "
                         "'attn' = --steps attention passes (rotating copies), 'copy' = "
                         "--steps plain copies of a 256 MiB tensor (the calibration kernel)")
    return ap.parse_args()


def source_digest():
    h = hashlib.sha256()
    for f in ("attention.hip", "common.hpp", "internal.hpp"):
        with open(os.path.join(ROOT, "block_verify_sv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(digest):
    """HBM bytes per attention pass from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "attention_qwen7b_25k_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"source_digest:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_pass:\s*([0-9]+)", text)
    if not m_src or not m_b or m_src.group(1) != digest:
        return None
    return int(m_b.group(1))


def cpu_baseline(seconds):
    """The float64 oracle on full verify cycles of the same workload, bounded in time."""
    import oracle
    import workloads as W
    from threadpoolctl import threadpool_info
    inp = W.make_workload_verify(WORKLOAD)
    g = W.make_workload_greedy(WORKLOAD)
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.verify_attention_ref(inp)
        oracle.accept_greedy_ref(g.logits, g.drafts, g.dtype)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 200:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": n / el, "unit": "cycles/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} full verify cycles ({WORKLOAD}: attention over 25,135 keys x 28 "
                      f"heads x 16 rows + greedy accept over 16 x 152,064), {el:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the verify path "
                                   "is built and measured on one GPU's share (it would shard "
                                   "by KV head, vocabulary or context); no figure at several "
                                   "GPUs is produced"}))
        sys.exit(2)
    import torch
    import block_verify_sv_amd as sv
    import workloads as W

    lib = sv.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.pmc_workload == "copy":
        src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_workload": "copy", "bytes_read": COPY_BYTES,
                          "bytes_written": COPY_BYTES, "launches": args.steps}), flush=True)
        return
    inp = W.make_workload_verify(WORKLOAD)
    g = W.make_workload_greedy(WORKLOAD)
    to_bf16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
        torch.bfloat16).to(dev)
    q = to_bf16(inp.q)
    k0, v0 = to_bf16(inp.k_cache), to_bf16(inp.v_cache)
    l0 = to_bf16(g.logits)
    R = max(1, args.copies)
    kcs = [k0] + [k0.clone() for _ in range(R - 1)]
    vcs = [v0] + [v0.clone() for _ in range(R - 1)]
    lgs = [l0] + [l0.clone() for _ in range(R - 1)]
    page_table = torch.from_numpy(inp.page_table).to(dev)
    ctx = torch.from_numpy(inp.ctx_lens).to(dev)
    drafts = torch.from_numpy(g.drafts).to(dev)
    B, K, Hq, D = inp.q.shape
    V = g.V
    desc = sv.make_desc(q, k0, page_table, int(inp.ctx_lens.max()), 0.0, args.split_keys,
                        int(inp.ctx_lens.sum()))
    ws_attn = torch.empty(sv.attention_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    n = ctypes.c_size_t()
    lib.sv_accept_greedy_workspace(B, K, V, ctypes.byref(n))
    ws_gr = torch.zeros(n.value, dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(B, K, Hq, dtype=torch.float32, device=dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    toks = torch.empty(B, K, dtype=torch.int32, device=dev)
    am = torch.empty(B, K, dtype=torch.int32, device=dev)
    stream = torch.cuda.Stream(device=dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    dref = ctypes.byref(desc)
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def attn(i):
        st = lib.sv_verify_attention(dref, P(q), P(kcs[i]), P(vcs[i]), P(page_table), P(ctx),
                                     None, P(out), P(lse), P(ws_attn), ws_attn.numel(), sp)
        if st:
            raise RuntimeError(lib.sv_last_error().decode())

    def accept(i):
        st = lib.sv_accept_greedy(B, K, V, sv.SV_BF16, P(lgs[i]), P(drafts), P(acc), P(toks),
                                  P(am), P(ws_gr), ws_gr.numel(), sp)
        if st:
            raise RuntimeError(lib.sv_last_error().decode())

    def cycle(i):
        attn(i)
        accept(i)

    if args.pmc_workload == "attn":
        with torch.cuda.stream(stream):
            for i in range(args.steps):
                attn(i % R)
        stream.synchronize()
        print(json.dumps({"pmc_workload": "attn", "passes": args.steps,
                          "kv_bytes": inp.kv_bytes(), "source_digest": source_digest()}),
              flush=True)
        return

    graphs = None
    with torch.cuda.stream(stream):
        for i in range(R):                      # first touch of every copy
            cycle(i)
        stream.synchronize()
        if args.launch == "graph":
            graphs = []
            for i in range(R):
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr, stream=stream):
                    cycle(i)
                graphs.append(gr)
            stream.synchronize()

        def step(i):
            if graphs is not None:
                graphs[i % R].replay()
            else:
                cycle(i % R)

        for i in range(args.warmup):
            step(i)
        stream.synchronize()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            step(i)
        e1.record(stream)
        e1.synchronize()
        torch.cuda.synchronize()
        ms_total = e0.elapsed_time(e1)

        # the attention pass alone, rotating copies, timed with events on its stream
        for i in range(20):
            attn(i % R)
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for i in range(args.attn_reps):
            attn(i % R)
        a1.record(stream)
        a1.synchronize()
        attn_us = a0.elapsed_time(a1) * 1000.0 / args.attn_reps

    ms_per_step = ms_total / args.steps
    kv_bytes = inp.kv_bytes()
    achieved = kv_bytes / (attn_us * 1e-6) / 1e9
    digest = source_digest()
    line = {
        "metric": "verify cycles/s (25k ctx, block 16, 1 MI355X); KV-read GB/s of the attention pass",
        "value": 1000.0 / ms_per_step,
        "unit": "cycles/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "B": B, "K": K, "Hq": Hq, "Hkv": inp.Hkv, "d": D,
                   "ctx": int(inp.ctx_lens[0]), "V": V, "page_size": inp.P,
                   "kv_copies": R, "launch": args.launch, "split_keys": args.split_keys},
        "kv_read_GBps": achieved,
        "kv_read_frac_of_peak": achieved / HBM_PEAK_GBPS,
        "roofline": {
            "kernel": "verify attention pass (attn_split_kernel + attn_merge_kernel)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": counter_traffic(digest),
            "algorithmic_bytes": kv_bytes,
            "avg_us": attn_us,
        },
        "source_digest": digest,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
