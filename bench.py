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
    ap.add_argument("--cpu-seconds", type=float, default=18.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the HBM read probe")
    ap.add_argument("--row", choices=["cycle", "hbm_probe"] + sorted(ROWS), default="cycle",
                    help="'cycle' (default) is the verify-cycle line; the others time one "
                         "further entry point on its own workload and print its own line; "
                         "'hbm_probe' times the hand-written streaming-read probe alone")
    ap.add_argument("--pmc-workload", choices=["attn", "copy"], default=None,
                    help="run a fixed loop for rocprofv3 --pmc counter passes and exit: "
                         "'attn' = --steps attention passes (rotating copies), 'copy' = "
                         "--steps plain copies of a 256 MiB tensor (the calibration kernel)")
    return ap.parse_args()


def source_digest():
    h = hashlib.sha256()
    for f in ("attention.hip", "attention.hpp", "limits.hpp", "common.hpp"):  # kernels + split plan
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


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(seconds, kv_bytes):
    """The float64 oracle on full verify cycles of the same workload, timed on the host's
    own cores after the GPU runs: one leg with the BLAS pool on every core the process
    may use, one with a single thread; each leg is the median of 3 timed runs of whole
    cycles, each run bounded to about seconds / 6."""
    import oracle
    import workloads as W
    from threadpoolctl import threadpool_info, threadpool_limits
    inp = W.make_workload_verify(WORKLOAD)
    g = W.make_workload_greedy(WORKLOAD)
    cores = len(os.sched_getaffinity(0))
    run_s = max(0.5, seconds / 6.0)

    def one_run():
        n = 0
        t0 = time.perf_counter()
        while True:
            oracle.verify_attention_ref(inp)
            oracle.accept_greedy_ref(g.logits, g.drafts, g.dtype)
            n += 1
            el = time.perf_counter() - t0
            if el >= run_s or n >= 100:
                return n, el

    legs = {}
    for name, threads in (("all_cores", cores), ("one_thread", 1)):
        with threadpool_limits(limits=threads):
            used = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
            runs = [one_run() for _ in range(3)]
        rates = sorted(n / el for n, el in runs)
        med = rates[1]
        legs[name] = {"cycles_per_s": med, "ms_per_cycle": 1000.0 / med,
                      "kv_GBps": kv_bytes * med / 1e9, "threads": int(used),
                      "runs": [{"cycles": n, "s": round(el, 3)} for n, el in runs]}
    blas = sorted({f"{i.get('internal_api')}:{i.get('threading_layer', '')}"
                   for i in threadpool_info()})
    a = legs["all_cores"]
    return {"value": a["cycles_per_s"], "unit": "cycles/s", "cores": cores, "kind": "oracle",
            "sample": f"median of 3 runs of whole verify cycles ({WORKLOAD}: float64 attention "
                      f"over 25,135 keys x 28 heads x 16 rows + greedy accept over 16 x "
                      f"152,064), each run ~{run_s:.1f} s; the all-cores leg is the value",
            "cpu_model": _cpu_model(), "blas": blas, "legs": legs}


# ------------------------------------------------------------------ HBM read probe
PROBE_WG_BYTES = (32 << 10, 64 << 10, 128 << 10, 256 << 10, 1 << 20)


def hbm_probe(torch, dev, single_bytes, copies, reps):
    """The hand-written streaming-read probe (libsvprobe.so): (1) one launch over 2 GiB,
    the chip's sustained read rate; (2) one launch over `single_bytes`, rotating over
    `copies` buffers (more than twice the last-level cache), timed exactly as the
    attention pass is (back-to-back launches between HIP events on the launch stream).
    Each figure is the best over a few workgroup sizes and both load kinds (ordinary and
    non-temporal)."""
    import block_verify_sv_amd as sv
    lib = ctypes.CDLL(os.path.join(os.path.dirname(sv.LIB_PATH), "libsvprobe.so"))
    lib.sv_probe_read.restype = ctypes.c_int
    lib.sv_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.sv_probe_workgroups.restype = ctypes.c_uint64
    lib.sv_probe_workgroups.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    big = 2 << 30
    big_buf = torch.ones(big // 2, dtype=torch.bfloat16, device=dev)
    bufs = [torch.ones(single_bytes // 2, dtype=torch.bfloat16, device=dev)
            for _ in range(copies)]
    max_wg = max(lib.sv_probe_workgroups(big, w) for w in PROBE_WG_BYTES)
    sink = torch.empty(int(max_wg) * 256 * 16, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(device=dev)
    sp = ctypes.c_void_p(stream.cuda_stream)

    def launch(buf, nbytes, wg, nt):
        st = lib.sv_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes, wg, nt,
                               ctypes.c_void_p(sink.data_ptr()), sp)
        if st:
            raise RuntimeError(f"sv_probe_read failed ({st})")

    def timed(fn, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            for i in range(3):
                fn(i)
            e0.record(stream)
            for i in range(n):
                fn(i)
            e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / n

    big_rows, single_rows = {}, {}
    for nt in (0, 1):
        for wg in PROBE_WG_BYTES:
            us = timed(lambda i: launch(big_buf, big, wg, nt), 10)
            big_rows[(wg, nt)] = big / (us * 1e-6) / 1e9
            us = timed(lambda i: launch(bufs[i % copies], single_bytes, wg, nt), reps)
            single_rows[(wg, nt)] = (us, single_bytes / (us * 1e-6) / 1e9)
    best_big = max(big_rows, key=big_rows.get)
    best_single = min(single_rows, key=lambda w: single_rows[w][0])
    del big_buf, bufs, sink
    torch.cuda.empty_cache()
    kind = ("ordinary", "non-temporal")
    return {"kernel": "hbm_read_kernel (libsvprobe.so, hand-written HIP)",
            "read_2GiB_GBps": big_rows[best_big], "read_2GiB_wg_bytes": best_big[0],
            "read_2GiB_loads": kind[best_big[1]],
            "single_launch_bytes": single_bytes,
            "single_launch_us": single_rows[best_single][0],
            "single_launch_GBps": single_rows[best_single][1],
            "single_launch_wg_bytes": best_single[0],
            "single_launch_loads": kind[best_single[1]],
            "sweep_GBps": {f"{w}{'/nt' if nt else ''}": [round(big_rows[(w, nt)], 1),
                                                        round(single_rows[(w, nt)][1], 1)]
                           for (w, nt) in big_rows}}


# ------------------------------------------------------------------ further rows
# name -> (workload, description, rotated copies = calls held by one graph)
ROWS = {
    "attn_batched": ("batched_paged", "verify attention, 8 sequences, log-uniform 4k-32k "
                     "contexts, shuffled 16-token pages", 3),
    "attn_72b": ("qwen72b_sampling", "verify attention, 72B geometry (64q/8kv, d 128), "
                 "ctx 25,000 + block 32", 6),
    "sample_72b": ("qwen72b_sampling", "sampling acceptance, block 32 over 152,064 "
                   "(target + draft logits)", 28),
    "compress": ("compressor_sar", "latent compressor, 32 images, D 4096, (C, N) = (64, 576)", 4),
    "compress_qwen": ("compressor_sar", "latent compressor, 32 images, D 4096, (C, N) = "
                      "(36, 324)", 4),
    "attn_tree60": ("qwen7b_tree60", "verify attention with the Tree-60 mask (61 nodes, 427 "
                    "rows per KV head), 7B layer, ctx 25,119", 12),
    "attn_drafter": ("vflash_drafter", "drafter block attention (one of its layers): anchor + "
                     "15 masks, bidirectional within the block, over ctx 25,119, 28q/4kv d128",
                     12),
    "attn_sar": ("compressor_sar", "semi-autoregressive block attention: 32 images x 5 slot "
                 "queries x 64 heads (d 64, fp16) over 64 compressed rows + the 5 slots, "
                 "bidirectional within the block", 15),
    "attn_sar_qwen": ("compressor_sar", "semi-autoregressive block attention: 32 images x 5 "
                      "slot queries x 64 heads (d 64, fp16) over 36 compressed rows + the 5 "
                      "slots, bidirectional within the block", 24),
    "tree60_accept": ("qwen7b_tree60", "greedy tree acceptance, 61 nodes over 152,064", 28),
    "tree60_sample": ("qwen7b_tree60", "sampling tree acceptance (recursive rejection), Tree-60 "
                      "over 152,064 (target + draft logits, T = 1)", 16),
    "commit_7b": ("qwen7b_25k", "cycle commit, 7B layer: the block's 16 K/V rows appended to "
                  "the paged cache (sv_kv_append), then the context-length and anchor update "
                  "(sv_commit); 32 calls per graph, inputs not rotated (64 KB)", 32),
    "lm_head": ("qwen7b_lmhead", "LM head fused with greedy acceptance: 16 x 3584 hidden "
                "states against the 152,064 x 3584 bf16 output embedding (1.09 GB, more than "
                "twice the Infinity Cache, so no rotation), packed once beforehand by "
                "sv_lm_head_pack (outside the timed region, as at model load)", 1),
    "lm_head_plain": ("qwen7b_lmhead", "LM head fused with greedy acceptance over the plain "
                      "[V][hidden] weight: 16 x 3584 hidden states against the 152,064 x 3584 "
                      "bf16 output embedding (1.09 GB, no rotation)", 1),
}


def graph_rounds(torch, stream, call, R, steps):
    """HIP graphs that replay exactly `steps` calls: one graph holding a call on each of
    the R rotated copies in turn (replayed steps // R times), plus one holding the first
    steps % R calls.  Returns [(graph, replays)]."""
    out = []
    for n, reps in ((R, steps // R), (steps % R, 1)):
        if n == 0 or reps == 0:
            continue
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=stream):
            for i in range(n):
                call(i, stream)
        out.append((gr, reps))
    return out


def run_row(args):
    """Time one further entry point on its workload: HIP graphs over rotated input copies
    on a side stream, HIP events around exactly --steps replays."""
    import torch
    import block_verify_sv_amd as sv
    import workloads as W
    sv.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl, desc_txt, R = ROWS[args.row]

    def dev_t(a, dtype):
        if dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(dev)
        if dtype == "f16":
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    flops = None
    if args.row.startswith("attn"):
        if args.row.startswith("attn_sar"):
            p = W.WORKLOADS[wl].params
            C = p["shapes"][0][0] if args.row == "attn_sar" else p["shapes"][1][0]
            inp = W.make_verify(W.rng_for(wl, 2000 + C), B=p["B"], K=p["S"], Hq=p["H"],
                                Hkv=p["H"], D=p["HD"], ctx_lens=[C] * p["B"], P=16,
                                dtype="f16", shuffle=True, mask=W.all_ones_mask(p["S"]))
        else:
            inp = W.make_workload_verify(wl)
        q = dev_t(inp.q, inp.dtype)
        ks = [dev_t(inp.k_cache, inp.dtype)]
        vs = [dev_t(inp.v_cache, inp.dtype)]
        ks += [ks[0].clone() for _ in range(R - 1)]
        vs += [vs[0].clone() for _ in range(R - 1)]
        pt, cl = i32(inp.page_table), i32(inp.ctx_lens)
        desc = sv.make_desc(q, ks[0], pt, int(inp.ctx_lens.max()), 0.0, 0, int(inp.ctx_lens.sum()))
        ws = torch.empty(sv.attention_workspace_bytes(desc), dtype=torch.uint8, device=dev)
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        nbytes = inp.kv_bytes()
        keys = int(inp.ctx_lens.sum()) + inp.B * inp.K
        flops = 4.0 * keys * inp.K * inp.Hq * inp.D    # QK^T and PV over every visible key
        shape = {"B": inp.B, "K": inp.K, "Hq": inp.Hq, "Hkv": inp.Hkv, "d": inp.D,
                 "ctx_sum": int(inp.ctx_lens.sum())}

        causal = np.array_equal(inp.mask, W.causal_mask(inp.K))
        mask = None if causal else sv.mask_array(inp.mask)

        def call(i, st):
            sv.verify_attention_into(desc, q, ks[i], vs[i], pt, cl, out, lse, mask, ws, st)
    elif args.row == "commit_7b":
        inp = W.make_workload_verify(wl)
        kc, vc = dev_t(inp.k_cache, inp.dtype), dev_t(inp.v_cache, inp.dtype)
        pt = i32(inp.page_table)
        start = i32(inp.ctx_lens)                 # the block goes to [ctx, ctx + K)
        rng = np.random.default_rng(0)
        new_rows = [dev_t(W.bf16_bits(rng.standard_normal((inp.B, inp.K, inp.Hkv, inp.D),
                                                          dtype=np.float32)), inp.dtype)
                    for _ in range(2)]
        acc = i32(np.full(inp.B, inp.K - 1))
        toks = i32(np.zeros((inp.B, inp.K)))
        ctx = i32(inp.ctx_lens)                   # grows by K per call; only commit reads it
        anchor = torch.empty(inp.B, dtype=torch.int32, device=dev)
        nbytes = 4 * new_rows[0].numel() * new_rows[0].element_size() + 16 * inp.B
        shape = {"B": inp.B, "K": inp.K, "Hkv": inp.Hkv, "d": inp.D}

        def call(i, st):
            sv.kv_append(new_rows[0], new_rows[1], start, pt, kc, vc, stream=st)
            sv.commit(acc, toks, ctx, anchor, stream=st)
    elif args.row == "tree60_accept":
        ti = W.make_workload_tree(wl)
        lg = [dev_t(ti.logits, ti.dtype)]
        lg += [lg[0].clone() for _ in range(R - 1)]
        par, tok = i32(ti.parents), i32(ti.tokens)
        outs = (torch.empty(ti.B, dtype=torch.int32, device=dev),
                torch.empty(ti.B, ti.K, dtype=torch.int32, device=dev),
                torch.empty(ti.B, ti.K, dtype=torch.int32, device=dev), None)
        sv.accept_greedy_tree(lg[0], par, tok, want_argmax=False, out=outs)
        nbytes = lg[0].numel() * lg[0].element_size()
        shape = {"B": ti.B, "K": ti.K, "V": ti.V}

        def call(i, st):
            sv.accept_greedy_tree(lg[i], par, tok, want_argmax=False, out=outs, stream=st)
    elif args.row == "tree60_sample":
        ts = W.make_workload_tree_sample(wl, 0)
        tl = [dev_t(ts.target_logits, ts.dtype)]
        dl = [dev_t(ts.draft_logits, ts.dtype)]
        tl += [tl[0].clone() for _ in range(R - 1)]
        dl += [dl[0].clone() for _ in range(R - 1)]
        tk = i32(ts.tokens)
        par = [int(x) for x in ts.parents]
        outs = (torch.empty(ts.B, dtype=torch.int32, device=dev),
                torch.empty(ts.B, ts.K, dtype=torch.int32, device=dev),
                torch.empty(ts.B, ts.K, dtype=torch.int32, device=dev))
        sv.accept_sample_tree(tl[0], dl[0], par, tk, ts.temperature, ts.seed, 0, out=outs)
        nbytes = (tl[0].numel() + dl[0].numel()) * tl[0].element_size()
        shape = {"B": ts.B, "K": ts.K, "V": ts.V, "T": ts.temperature}

        def call(i, st):
            sv.accept_sample_tree(tl[i], dl[i], par, tk, ts.temperature, ts.seed, i, out=outs,
                                  stream=st)
    elif args.row in ("lm_head", "lm_head_plain"):
        li = W.make_workload_lm_head(wl)
        hs = dev_t(li.hidden_states, li.dtype)
        wt = dev_t(li.weight, li.dtype)
        dr = i32(li.drafts)
        outs = (torch.empty(li.B, dtype=torch.int32, device=dev),
                torch.empty(li.B, li.K, dtype=torch.int32, device=dev), None)
        nbytes = (wt.numel() + hs.numel()) * 2
        flops = 2.0 * li.B * li.K * li.V * li.hidden
        shape = {"B": li.B, "K": li.K, "hidden": li.hidden, "V": li.V}
        if args.row == "lm_head":
            wp = sv.lm_head_pack(wt)
            del wt

            def call(i, st):
                sv.lm_head_greedy_packed(hs, wp, li.V, dr, want_argmax=False, out=outs,
                                         stream=st)
        else:
            def call(i, st):
                sv.lm_head_greedy(hs, wt, dr, want_argmax=False, out=outs, stream=st)
        call(0, None)
    elif args.row == "sample_72b":
        smp = W.make_workload_sample(wl, 0)
        tl = [dev_t(smp.target_logits, smp.dtype)]
        dl = [dev_t(smp.draft_logits, smp.dtype)]
        tl += [tl[0].clone() for _ in range(R - 1)]
        dl += [dl[0].clone() for _ in range(R - 1)]
        dr = i32(smp.drafts)
        acc = torch.empty(smp.B, dtype=torch.int32, device=dev)
        toks = torch.empty(smp.B, smp.K, dtype=torch.int32, device=dev)
        sv.accept_sample(tl[0], dl[0], dr, smp.temperature, smp.seed, 0, out=(acc, toks))
        nbytes = (tl[0].numel() + dl[0].numel()) * tl[0].element_size()
        shape = {"B": smp.B, "K": smp.K, "V": smp.V, "T": smp.temperature}

        def call(i, st):
            sv.accept_sample(tl[i], dl[i], dr, smp.temperature, smp.seed, i, out=(acc, toks),
                             stream=st)
    else:
        p = W.WORKLOADS[wl].params
        C, N = p["shapes"][0] if args.row == "compress" else p["shapes"][1]
        ci = W.make_compress(W.rng_for(wl, 0), B=p["B"], C=C, N=N, D=p["D"])
        qd = dev_t(ci.queries, "f16")
        fs = [dev_t(ci.feats, "f16")]
        fs += [fs[0].clone() for _ in range(R - 1)]
        out = torch.empty(ci.B, C, ci.D, dtype=torch.float16, device=dev)
        sv.latent_compress(qd, fs[0], 1.0, out=out)
        nbytes = (fs[0].numel() + qd.numel() + out.numel()) * 2
        flops = 4.0 * ci.B * C * N * ci.D
        shape = {"B": ci.B, "C": C, "N": N, "D": ci.D}

        def call(i, st):
            sv.latent_compress(qd, fs[i], 1.0, out=out, stream=st)

    stream = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(stream):
        for i in range(R):
            call(i, stream)
        stream.synchronize()
        rounds = graph_rounds(torch, stream, call, R, args.steps)
        for _ in range(max(1, args.warmup // R)):
            rounds[0][0].replay()
        stream.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for gr, reps in rounds:
            for _ in range(reps):
                gr.replay()
        e1.record(stream)
        e1.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / args.steps
    gbps = nbytes / (us * 1e-6) / 1e9
    line = {"row": args.row, "workload": wl, "what": desc_txt, "config": shape,
            "us_per_call": us, "calls_per_s": 1e6 / us, "algorithmic_bytes": int(nbytes),
            "GBps": gbps, "frac_of_hbm_peak": gbps / HBM_PEAK_GBPS, "steps": args.steps,
            "warmup": args.warmup, "calls_per_graph": R,
            "rotated_copies": 1 if args.row == "commit_7b" else R}
    if flops is not None:
        line["TFLOPs"] = flops / (us * 1e-6) / 1e12
        line["flops_per_call"] = flops
    print(json.dumps(line), flush=True)


def run_hbm_probe(args):
    """The hand-written HIP read probe alone (its own JSON line)."""
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    import workloads as W
    kv = W.make_workload_verify(WORKLOAD).kv_bytes()
    line = {"row": "hbm_probe"}
    line.update(hbm_probe(torch, dev, kv, max(1, args.copies), args.attn_reps))
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.row == "hbm_probe":
        run_hbm_probe(args)
        return
    if args.row != "cycle":
        if args.gpus != 1:
            print(json.dumps({"error": "one GPU only"}))
            sys.exit(2)
        run_row(args)
        return
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

    with torch.cuda.stream(stream):
        for i in range(R):                      # first touch of every copy
            cycle(i)
        stream.synchronize()
        if args.launch == "graph":
            # graphs of R cycles (one per rotated copy) replayed back to back, plus a
            # remainder graph, so exactly --steps cycles run in the timed region
            rounds = graph_rounds(torch, stream, lambda i, st: cycle(i), R, args.steps)
            warm = graph_rounds(torch, stream, lambda i, st: cycle(i), R, args.warmup)
            stream.synchronize()

            def run_all(rs):
                for gr, reps in rs:
                    for _ in range(reps):
                        gr.replay()
        else:
            def run_all(n):
                for i in range(n):
                    cycle(i % R)
            rounds, warm = args.steps, args.warmup

        run_all(warm)
        stream.synchronize()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run_all(rounds)
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
    probe = None if args.no_probe else hbm_probe(torch, dev, kv_bytes, R, args.attn_reps)
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
    if probe is not None:
        line["achievable"] = probe
        line["roofline"]["achievable_GBps"] = probe["single_launch_GBps"]
        line["roofline"]["frac_of_achievable"] = achieved / probe["single_launch_GBps"]
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds, kv_bytes)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
