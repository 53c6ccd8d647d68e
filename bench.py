"""Benchmark of one absorbed-MLA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--splits S]
                    [--pages-per-split P]
                    [--no-cpu-baseline] [--flush] [--no-graph]

A step is the whole hot path over one batch of synthetic input already resident
in HBM: mla_absorb_q -> mla_decode_paged -> mla_combine -> mla_up_v, all on the
current HIP stream; the last two run as one launch (mla_combine_up_v) where its fused
kernel covers the shape.

Timing (default).  The step's inputs, outputs and workspace exist in n copies (n >= 2,
enough that n steps read more than twice the 256 MB Infinity Cache), used in turn,
so a step never finds its cache pages, weights or queries in L2 or the MALL: every
step starts from HBM, as a decode step that reads another layer's cache does.  After
W warmup steps over every copy, exactly K steps run back to back over the copies
(HIP graphs of up to 8 steps, replayed) in one region between two synchronizations
and two HIP events; the step time is that region's time / K.  Back-to-back replay is
how a serving loop runs the step; timing each step alone between two events would
add the event and graph-launch latency (about 10 us here) to every step.  Per-call
times (and the decode kernel's time in the roofline object) are measured the same
way, each call alone back to back over the copies (median of 5 runs of about K
calls), and agree with rocprofv3's kernel durations.  --no-graph launches the same
sequences eagerly.  --flush keeps the earlier method: one copy, a 1 GiB read-only
cache flush before every step, each step between its own events.

Prints one JSON line.  `value` is the algorithmic TFLOP/s of the whole step
(attention flops of the absorbed method plus the two projections, divided by the
step time); the line also carries latent-KV GB/s, sequences/s, the roofline
object of the dominant kernel (the split-KV decode), the roofline fractions of the
attention calls (decode + merge) and of the whole step against the nominal 8 TB/s
and against a measured 1 GiB device copy (`roofline_path`), and the CPU oracle
baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode attention TFLOP/s + latent-KV GB/s (% MI355X roofline), seqs/s"
HEADLINE = "ragged_b64"
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20  # Infinity Cache of one MI355X
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode.json")
CSRC = os.path.join(ROOT, "mla_latent_kv_09_amd", "csrc")
KERNEL_SRC = {"decode_mfma_kernel": "decode_mfma.hip", "decode_m32_kernel": "decode_m32.hip",
              "decode_m32_kernel_fp8": "decode_m32.hip", "decode_m32_kernel_mxfp4": "decode_m32.hip",
              "decode_generic_kernel": "kernels_generic.hip",
              "prefill_attn_kernel": "prefill.hip", "decompress_kernel": "prefill.hip"}


def cache_row_bytes(cfg, kv_dtype="bf16"):
    """Bytes one token occupies in the latent cache: d_c + d_R elements of the storage
    type; for the FP8 cache d_c E4M3 codes, d_R bf16 and one float32 scale; for the MXFP4
    cache d_c / 2 bytes of codes, d_R bf16 and d_c / 32 scale bytes."""
    if kv_dtype == "fp8":
        return cfg.d_c + 2 * cfg.d_R + 4
    if kv_dtype == "mxfp4":
        return cfg.d_c // 2 + 2 * cfg.d_R + cfg.d_c // 32
    return (cfg.d_c + cfg.d_R) * (2 if cfg.dtype == "bf16" else 4)


def algorithmic_work(cfg, seq_lens, q_lens, kv_dtype="bf16"):
    """(attention flops, projection flops, latent-KV bytes, weight bytes) of one step.

    Per (query row, visible key): 2*(d_c/G + d_R) flops for the score and 2*d_c/G for
    P.c_KV.  Latent rows are counted once per sequence (cache_row_bytes each).  The two
    projections are 2*T*H*d_hc*d_c/G flops each.
    """
    d_cg = cfg.d_c // cfg.groups
    elem = 2 if cfg.dtype == "bf16" else 4
    row_bytes = cache_row_bytes(cfg, kv_dtype)
    per_key = cfg.heads * (2 * (d_cg + cfg.d_R) + 2 * d_cg)
    att = 0
    kv_bytes = 0
    for L, q in zip(seq_lens, q_lens):
        L, q = int(L), int(q)
        for i in range(q):
            att += per_key * (L - q + i + 1 if cfg.causal else L)
        kv_bytes += L * row_bytes
    T = int(sum(q_lens))
    proj = 2 * (2 * T * cfg.heads * cfg.d_hc * d_cg)
    w_bytes = 2 * cfg.heads * cfg.d_hc * d_cg * elem
    return att, proj, kv_bytes, w_bytes


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel, workload, splits):
    """HBM bytes per launch from committed rocprofv3 counters (one record per kernel and
    workload), if they were taken on this kernel, its current source, this workload and
    this split count (1 for the prefill kernels, which do not split)."""
    try:
        with open(TRAFFIC_FILE) as f:
            recs = json.load(f).get("records", [])
    except (OSError, ValueError, AttributeError):
        return None
    for rec in recs:
        if rec.get("kernel") != kernel or rec.get("workload") != workload:
            continue
        if rec.get("num_splits") != splits:
            continue
        if rec.get("kernel_source_sha256_16") != source_hash(os.path.join(CSRC, KERNEL_SRC[kernel])):
            continue
        return rec.get("bytes_per_launch")
    return None


def cpu_baseline(w, att_flops_full, min_s=10.0):
    """Time the fp64 oracle on a bounded sample of the same workload (whole heads of
    sequences taken in order, starting over at the first once all are done, until just
    past min_s seconds of CPU work; one sequence of the longest workload takes about
    that) and scale to the step's algorithmic TFLOP/s."""
    import numpy as np  # noqa: F401
    import oracle.mla_oracle as om

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    B = len(w.latents)
    done_seqs = []
    t_spent = 0.0
    t0 = time.perf_counter()
    while True:
        b = len(done_seqs) % B
        tb = time.perf_counter()
        om.mla_decode(w.q_c, w.q_r, w.latents, w.w_uk, w.w_uv, w.cu_q, groups=w.cfg.groups,
                      rope_base=w.cfg.rope_base, causal=w.cfg.causal, seq_subset=[b])
        t_spent += time.perf_counter() - tb
        done_seqs.append(b)
        elapsed = time.perf_counter() - t0
        if elapsed > min_s:
            break
    sub_lens = [w.seq_lens[b] for b in done_seqs]
    sub_q = [w.q_lens[b] for b in done_seqs]
    att, proj, _, _ = algorithmic_work(w.cfg, sub_lens, sub_q)
    tflops = (att + proj) / t_spent / 1e12
    passes = len(done_seqs) / B
    return {
        "value": tflops, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "seqs_per_s": len(done_seqs) / t_spent,
        "sample": f"{len(done_seqs)} sequence decodes ({passes:.2f} passes over the {B} "
                  f"sequences, all heads) of {w.cfg.name}, fp64 non-absorbed numpy oracle, "
                  f"{t_spent:.1f} s",
    }


def step_calls(step):
    """(name, DecodeStep method) of the calls one step issues: the merge and W_UV are one
    launch (mla_combine_up_v) where the fused kernel covers the shape."""
    calls = [("absorb_q", "absorb"), ("decode_paged", "attend")]
    if step.fused:
        return calls + [("combine_up_v", "merge_project")]
    return calls + [("combine", "merge"), ("up_v", "project")]


def flush_timing(args, w, torch, harness, stream):
    """The earlier method, kept for comparison (--flush): one input copy, a 1 GiB
    read-only flush before every step, events around each step and between the calls
    of a second pass."""
    d = harness.to_device(w)
    step = harness.make_step(w, d, args.splits, args.pages_per_split, keep_latent=args.keep_latent)
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")

    calls = step_calls(step)

    def one_step(ev=None):
        if ev is None:
            step()
            return
        ev[0].record(stream)
        for i, (_, attr) in enumerate(calls):
            getattr(step, attr)()
            ev[i + 1].record(stream)

    for _ in range(args.warmup):
        flush_buf.max()
        one_step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
              for _ in range(args.steps)]
    for k in range(args.steps):
        flush_buf.max()
        one_step(events[k])
    torch.cuda.synchronize()
    parts = {name: statistics.median([e[i].elapsed_time(e[i + 1]) for e in events])
             for i, (name, _) in enumerate(calls)}
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
    ev_step = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    wall0 = time.perf_counter()
    for k in range(args.steps):
        flush_buf.max()
        ev_step[k][0].record(stream)
        if graph is not None:
            graph.replay()
        else:
            step()
        ev_step[k][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = statistics.median(e[0].elapsed_time(e[1]) for e in ev_step)
    return ms, parts, parts["decode_paged"], step.num_splits, step, wall, graph is not None


def measure_copy_gbps(torch, stream, mib=1024, reps=5):
    """Achievable HBM streaming rate on this GPU: a 1 GiB device-to-device copy (read +
    write bytes / time), median of `reps`, the same bytes counted both ways."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del src, dst
    return 2 * (mib << 20) / (statistics.median(times) * 1e-3) / 1e9


def path_roofline(att, proj, kv_bytes, w_bytes, parts, step_ms, peak_tflops, copy_gbps):
    """Roofline fractions of the attention calls (decode + merge) and of the whole step
    (all four calls): the binding roof's time, max(bytes / bandwidth, flops / peak), over the
    measured time, against the nominal 8 TB/s and against the measured copy rate."""
    def frac(flops, nbytes, ms, gbps):
        t_roof = max(nbytes / (gbps * 1e9), flops / (peak_tflops * 1e12))
        return t_roof / (ms * 1e-3)
    # decode + merge; a fused merge launch also carries the value projection
    att_ms = parts["decode_paged"] + parts.get("combine", parts.get("combine_up_v", 0.0))
    return {
        "hbm_copy_gbps": copy_gbps,
        "attention": {"ms": att_ms, "frac": frac(att, kv_bytes, att_ms, HBM_PEAK_GBPS),
                      "frac_of_copy_bw": frac(att, kv_bytes, att_ms, copy_gbps)},
        "step": {"ms": step_ms, "frac": frac(att + proj, kv_bytes + w_bytes, step_ms, HBM_PEAK_GBPS),
                 "frac_of_copy_bw": frac(att + proj, kv_bytes + w_bytes, step_ms, copy_gbps)},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=HEADLINE)
    ap.add_argument("--splits", type=int, default=None,
                    help="split count instead of the planner's (each sequence cut into S equal "
                         "parts unless --pages-per-split is given)")
    ap.add_argument("--pages-per-split", type=int, default=0,
                    help="with --splits: fixed split length in pages")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush", action="store_true",
                    help="one input copy and a 1 GiB read-only cache flush before every step, "
                         "each step timed alone (the earlier method) instead of rotating copies")
    ap.add_argument("--no-graph", action="store_true", help="launch the calls eagerly")
    ap.add_argument("--threshold", type=int, default=256,
                    help="query rows at which the library's dispatch takes the decompressed "
                         "branch (batches whose largest q_len reaches it, e.g. --config "
                         "prefill_b8_l4096)")
    ap.add_argument("--kv-dtype", choices=["bf16", "fp8", "mxfp4"], default="bf16",
                    help="latent cache format: bf16 rows (default), FP8 E4M3 pages written by "
                         "mla_append_kv_fp8 or MXFP4 pages written by mla_append_kv_mxfp4 (a "
                         "separate line, never the headline)")
    ap.add_argument("--keep-latent", action="store_true",
                    help="have a fused merge launch also write the merged latent rows (the "
                         "step's output is out and lse either way)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the decode path is built "
              "and measured on a single MI355X", file=sys.stderr)
        sys.exit(2)

    import torch

    from mla_latent_kv_09_amd import harness, mla
    from mla_latent_kv_09_amd import workloads as wl

    if not torch.cuda.is_available():
        print("no GPU visible: bench.py needs an MI355X", file=sys.stderr)
        sys.exit(1)
    mla.load()  # fails loudly when the HIP library is missing

    cfg = wl.CONFIGS[args.config]
    w = wl.make_workload(cfg)
    if args.kv_dtype != "bf16" and args.flush:
        print("a quantized cache takes the default (rotated copies) timing", file=sys.stderr)
        sys.exit(2)
    att, proj, kv_bytes, w_bytes = algorithmic_work(cfg, w.seq_lens, w.q_lens, args.kv_dtype)
    stream = torch.cuda.current_stream()
    if mla.branch(w.q_lens.tolist(), args.threshold) == mla.BRANCH_DECOMPRESSED:
        if args.kv_dtype != "bf16" or args.flush:
            print("the decompressed branch takes the bf16 cache and the default timing", file=sys.stderr)
            sys.exit(2)
        print(json.dumps(prefill_bench(args, w, torch, harness, mla, stream)))
        return

    if not args.flush:
        # Rotation: n_copies independent device copies of the step's inputs, outputs and
        # workspace, used in turn, so every step reads data that the steps since its
        # copy's last use (together more than twice the 256 MB Infinity Cache) have
        # evicted from L2 and MALL: each step starts from HBM.  Steps and calls are
        # timed back to back inside HIP graphs, as a serving loop runs them.
        n_copies = max(2, min(8, math.ceil(2 * MALL_BYTES / (kv_bytes + w_bytes))))
        steps = [harness.make_step(w, device_copy(w, harness, args.kv_dtype), args.splits,
                                   args.pages_per_split, keep_latent=args.keep_latent)
                 for _ in range(n_copies)]
        step = steps[0]
        S = step.num_splits
        per_graph = n_copies * max(1, math.ceil(8 / n_copies))  # calls captured per graph

        def graph_of(calls):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for c in calls:
                    c()
            g.replay()
            torch.cuda.synchronize()
            return g

        def runner(calls):
            """A callable that issues `calls` once: a graph replay, or eager launches."""
            if args.no_graph:
                return lambda: [c() for c in calls]
            return graph_of(calls).replay

        def timed(run, reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                run()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1)

        for _ in range(max(1, args.warmup)):
            for st in steps:
                st()
        torch.cuda.synchronize()
        # Per-call times: each call alone, back to back over the rotated copies (median of
        # 5 runs of about K calls).
        reps = max(1, math.ceil(args.steps / per_graph))
        parts = {}
        for name, attr in step_calls(step):
            run = runner([getattr(steps[i % n_copies], attr) for i in range(per_graph)])
            parts[name] = statistics.median(timed(run, reps) / (reps * per_graph) for _ in range(5))
            del run
        dec = parts["decode_paged"]
        append = measure_append(args, w, torch, harness, mla, wl, steps, runner, timed, reps,
                                per_graph)
        # Step time: exactly K whole steps back to back over the rotated copies, one timed
        # region between two synchronizations.
        full, rest = divmod(args.steps, per_graph)
        run_full = runner([steps[i % n_copies] for i in range(per_graph)]) if full else None
        run_rest = runner([steps[i % n_copies] for i in range(rest)]) if rest else None

        def k_steps():
            for _ in range(full):
                run_full()
            if run_rest is not None:
                run_rest()

        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        ms = timed(k_steps, 1) / args.steps
        wall = time.perf_counter() - wall0
        timing = {"method": "rotate", "copies": n_copies, "steps_per_graph": per_graph}
        graph_used = not args.no_graph
    else:
        ms, parts, dec, S, step, wall, graph_used = flush_timing(args, w, torch, harness, stream)
        timing = {"method": "flush"}
        append = None

    copy_gbps = measure_copy_gbps(torch, stream)
    flops = att + proj
    tflops = flops / (ms * 1e-3) / 1e12
    kv_gbps = kv_bytes / (ms * 1e-3) / 1e9
    seqs = cfg.batch / (ms * 1e-3)

    # Dominant kernel: split-KV decode.  Bound by whichever roof is further away.
    peak_f = BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else FP32_PEAK_TFLOPS
    t_hbm = kv_bytes / (HBM_PEAK_GBPS * 1e9)
    t_mfma = att / (peak_f * 1e12)
    kernel = decode_kernel_name(cfg, int(w.total_q), S, args.kv_dtype,
                                torch.cuda.get_device_properties(0).multi_processor_count)
    traffic = measured_traffic(kernel, cfg.name, S)
    if t_hbm >= t_mfma:
        achieved = kv_bytes / (dec * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic}
    else:
        achieved = att / (dec * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak_f, "unit": "TFLOP/s",
                "frac": achieved / peak_f, "traffic": traffic}
    roof.update({"kernel": kernel, "kernel_ms": dec, "algorithmic_bytes": kv_bytes, "algorithmic_flops": att})

    out = {
        "metric": METRIC, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "kv_cache": {"fp8": "fp8_e4m3", "mxfp4": "mxfp4"}.get(args.kv_dtype, cfg.dtype),
                   "batch": cfg.batch, "heads": cfg.heads, "d_hc": cfg.d_hc,
                   "d_c": cfg.d_c, "d_R": cfg.d_R, "groups": cfg.groups, "page_size": cfg.page_size,
                   "seq_len": cfg.seq_len, "seq_len_range": cfg.seq_len_range,
                   "total_q": int(w.total_q), "num_splits": S,
                   "pages_per_split": step.pages_per_split, "timing": timing,
                   "merge_and_up_v": "one launch" if step.fused else "two launches",
                   "hip_graph": graph_used},
        "latent_kv_gbps": kv_gbps, "latent_kv_frac_hbm_peak": kv_gbps / HBM_PEAK_GBPS,
        "tflops_frac_mfma_peak": tflops / peak_f, "seqs_per_s": seqs,
        "roofline_path": path_roofline(att, proj, kv_bytes, w_bytes, parts, ms, peak_f, copy_gbps),
        "kernel_ms": parts, "wall_s_timed_region": wall,
        "roofline": roof,
    }
    if append is not None:
        out["append_kv"] = append
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, att)
    print(json.dumps(out))


def measure_append(args, w, torch, harness, mla, wl, steps, runner, timed, reps, per_graph):
    """The latent-cache append (mla_append_kv, the call before the decode; not part of the
    step): (1) this workload's T new rows per call, back to back over the rotated copies;
    (2) a prefill-shaped bulk append that writes every slot of the first sequences (at
    most 65536 rows; q_len = seq_len, so each sequence's rows 0 .. L-1), rotated over the
    copies like the step, whose bytes (each row read once and written once in the cache's
    format) give the kernel's HBM roofline.  With --kv-dtype fp8 / mxfp4 the call is
    mla_append_kv_fp8 / mla_append_kv_mxfp4, which also quantizes the latent."""
    cfg = w.cfg
    elem = 2 if cfg.dtype == "bf16" else 4
    kv_dtype = args.kv_dtype
    append = {"fp8": mla.append_kv_fp8, "mxfp4": mla.append_kv_mxfp4}.get(kv_dtype, mla.append_kv)
    n = len(steps)
    new = wl.make_new_tokens(w)
    tensors = [harness.new_tokens_to_device(w, new, st.kv.device) for st in steps]

    def call(i):
        st, (c, k) = steps[i % n], tensors[i % n]
        return lambda: append(c, k, st.kv, st.page_table, st.seq_lens, st.cu_q, rope=st.rope)

    run = runner([call(i) for i in range(per_graph)])
    ms_t = statistics.median(timed(run, reps) / (reps * per_graph) for _ in range(5))
    del run
    res = {"rows": int(w.total_q), "ms": ms_t}
    if cfg.seq_len is None:  # bulk case only for equal lengths
        return res
    L, B = int(cfg.seq_len), cfg.batch
    nb = max(1, min(B, 65536 // L))  # whole sequences, at most 65536 rows
    bulk = wl.make_new_tokens(w, rows=nb * L)
    cu = torch.tensor([min(b, nb) * L for b in range(B + 1)], dtype=torch.int32,
                      device=steps[0].kv.device)
    bulk_t = [harness.new_tokens_to_device(w, bulk, st.kv.device) for st in steps]

    def bulk_call(i):
        st, (c, k) = steps[i % n], bulk_t[i % n]
        return lambda: append(c, k, st.kv, st.page_table, st.seq_lens, cu, rope=st.rope)

    run = runner([bulk_call(i) for i in range(n)])
    bulk_reps = max(2, min(10, reps))
    ms_b = statistics.median(timed(run, bulk_reps) / (bulk_reps * n) for _ in range(5))
    del run, bulk_t
    # each row read once (bf16 or fp32 inputs) and written once in the cache's format
    nbytes = nb * L * ((cfg.d_c + cfg.d_R) * elem + cache_row_bytes(cfg, kv_dtype))
    gbps = nbytes / (ms_b * 1e-3) / 1e9
    res["bulk"] = {"rows": nb * L, "ms": ms_b, "algorithmic_bytes": nbytes, "gbps": gbps,
                   "frac_hbm_peak": gbps / HBM_PEAK_GBPS}
    return res


def prefill_work(cfg, seq_lens, q_lens):
    """(attention flops, decompression flops, latent-KV bytes, workspace bytes) of the
    decompressed branch: per (query row, visible key, head) 2 (d_hc + d_R) + 2 d_hc flops;
    per cache row and head 2 * 2 d_c d_hc flops for K and V; the workspace (K and V of
    every row, bf16) written once and read back once."""
    per_key = cfg.heads * (2 * (cfg.d_hc + cfg.d_R) + 2 * cfg.d_hc)
    att = dec = kv = 0
    for L, q in zip(seq_lens, q_lens):
        L, q = int(L), int(q)
        for i in range(q):
            att += per_key * (L - q + i + 1 if cfg.causal else L)
        dec += L * cfg.heads * 2 * 2 * cfg.d_c * cfg.d_hc
        kv += L * (cfg.d_c + cfg.d_R) * 2
    ws = sum(int(L) for L in seq_lens) * cfg.heads * cfg.d_hc * 2 * 2
    return att, dec, kv, ws


def prefill_bench(args, w, torch, harness, mla, stream):
    """The decompressed branch (mla_decompress_kv + mla_prefill_attention), timed like the
    decode step (two device copies, used in turn, back to back in HIP graphs), plus the
    four absorbed calls on the same inputs for the dispatch comparison (fewer steps: the
    absorbed form of a prompt is several times slower)."""
    cfg = w.cfg
    att, dec, kv_bytes, ws_bytes = prefill_work(cfg, w.seq_lens, w.q_lens)
    steps = [harness.make_step(w, harness.to_device(w), threshold=args.threshold) for _ in range(2)]

    def timed(calls, reps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in calls:
                c()
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * len(calls))

    for _ in range(max(1, args.warmup)):
        for st in steps:
            st()
    torch.cuda.synchronize()
    reps = max(1, math.ceil(args.steps / 2))
    parts = {
        "decompress_kv": statistics.median(timed([steps[0].decompress, steps[1].decompress], reps)
                                           for _ in range(3)),
        "prefill_attention": statistics.median(timed([steps[0].prefill_attend, steps[1].prefill_attend],
                                                     reps) for _ in range(3)),
    }
    wall0 = time.perf_counter()
    full, rest = divmod(args.steps, 2)
    ms = (timed([steps[0], steps[1]], full) * 2 * full + (timed([steps[0]], rest) * rest if rest else 0.0)) / args.steps
    wall = time.perf_counter() - wall0
    # The absorbed calls on the first copy (a step without a threshold never dispatches).
    d0 = harness.DeviceWorkload(q_c=steps[0].q_c, q_r=steps[0].q_r, w_uk=steps[0].w_uk,
                                w_uv=steps[0].w_uv, kv=steps[0].kv, page_table=steps[0].page_table,
                                seq_lens=steps[0].seq_lens, cu_q=steps[0].cu_q, rope=steps[0].rope)
    absorbed = harness.make_step(w, d0)
    absorbed()
    torch.cuda.synchronize()
    abs_reps = max(2, min(10, args.steps // 20))
    abs_ms = statistics.median(timed([absorbed], abs_reps) for _ in range(3))
    abs_att, abs_proj, _, _ = algorithmic_work(cfg, w.seq_lens, w.q_lens)
    del absorbed
    t_att = parts["prefill_attention"]
    achieved = att / (t_att * 1e-3) / 1e12
    return {
        "metric": METRIC, "value": (att + dec) / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "branch": "decompressed", "threshold": args.threshold,
                   "batch": cfg.batch, "heads": cfg.heads, "d_hc": cfg.d_hc, "d_c": cfg.d_c,
                   "d_R": cfg.d_R, "q_len": cfg.q_len, "seq_len": cfg.seq_len,
                   "total_q": int(w.total_q), "timing": {"method": "rotate", "copies": 2}},
        "kernel_ms": parts, "wall_s_timed_region": wall,
        "seqs_per_s": cfg.batch / (ms * 1e-3),
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS,
                     "traffic": measured_traffic("prefill_attn_kernel", cfg.name, 1),
                     "kernel": "prefill_attn_kernel", "kernel_ms": t_att, "algorithmic_flops": att},
        "decompress": {"ms": parts["decompress_kv"], "algorithmic_flops": dec,
                       "tflops": dec / (parts["decompress_kv"] * 1e-3) / 1e12,
                       "traffic": measured_traffic("decompress_kernel", cfg.name, 1),
                       "workspace_bytes": ws_bytes, "latent_kv_bytes": kv_bytes},
        "absorbed_branch": {"ms_per_step": abs_ms, "algorithmic_flops": abs_att + abs_proj,
                            "speedup_of_dispatch": abs_ms / ms},
    }


def device_copy(w, harness, kv_dtype):
    """One device copy of the workload; with kv_dtype fp8 / mxfp4 its cache replaced by
    pages of that format that the library's append writes from the bf16 rows (the bf16
    pool is freed)."""
    d = harness.to_device(w)
    if kv_dtype in ("fp8", "mxfp4"):
        d.kv = harness.quant_pool_by_append(w, d, kv_dtype)
    return d


def decode_kernel_name(cfg, total_q, num_splits, kv_dtype="bf16", cu_count=256):
    """The decode kernel the library dispatches for this shape (same rule as the library:
    MLA_KV_DECODE_KERNEL = generic / mfma / mfma128 / mfma64 / mfma32[-128|-64]; by default, for one
    latent group, the 32x32x16 kernel when one workgroup per (token, split) fills the
    device and the 16x16x32 kernel's 64-head split otherwise)."""
    mfma_shape = (cfg.dtype == "bf16" and cfg.heads == 128 and cfg.groups in (1, 2)
                  and cfg.d_c == 512 and cfg.d_R == 64 and cfg.page_size == 64)
    choice = os.environ.get("MLA_KV_DECODE_KERNEL", "")
    if kv_dtype in ("fp8", "mxfp4"):  # one kernel form over quantized pages
        return "decode_m32_kernel_" + kv_dtype
    if choice == "generic" or not mfma_shape:
        return "decode_generic_kernel"
    if cfg.groups != 1 or choice in ("mfma128", "mfma64"):
        return "decode_mfma_kernel"
    # The library's rule for one latent group: two 64-head workgroups per (token, split)
    # when 2 * total_q * num_splits fits the compute units.
    head_split = 2 if 2 * total_q * num_splits <= cu_count else 1
    if choice.startswith("mfma32") or head_split == 1:
        return "decode_m32_kernel"
    return "decode_mfma_kernel"


if __name__ == "__main__":
    main()
