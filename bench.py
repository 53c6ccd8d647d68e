"""Benchmark of one absorbed-MLA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--splits S]
                    [--no-cpu-baseline] [--no-flush]

A step is the whole hot path over one batch of synthetic input already resident
in HBM: mla_absorb_q -> mla_decode_paged -> mla_combine -> mla_up_v, all on the
current HIP stream, captured once as a HIP graph and replayed (--no-graph
launches the four calls eagerly).  Before every timed step a 1 GiB buffer is
read (a max-reduction) so the L2 and the 256 MB Infinity Cache hold nothing of the
step's working set (a real decode step reads a different layer's cache every
time).  The flush only reads: a flush that writes leaves up to 256 MB of dirty
lines whose write-back then competes with the step's own reads.
Each step is bracketed by HIP events; the reported time is the median over the
K timed steps.  Per-kernel times (and the decode kernel's time in the roofline
object) come from a second pass of K eager steps with events between the calls.

Prints one JSON line.  `value` is the algorithmic TFLOP/s of the whole step
(attention flops of the absorbed method plus the two projections, divided by the
step time); the line also carries latent-KV GB/s, sequences/s, the roofline
object of the dominant kernel (the split-KV decode) and the CPU oracle baseline.
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
HEADLINE = "dsv3_b16_l4096"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode.json")
CSRC = os.path.join(ROOT, "mla_latent_kv_09_amd", "csrc")
KERNEL_SRC = {"decode_mfma_kernel": "decode_mfma.hip",
              "decode_generic_kernel": "kernels_generic.hip"}


def algorithmic_work(cfg, seq_lens, q_lens):
    """(attention flops, projection flops, latent-KV bytes, weight bytes) of one step.

    Per (query row, visible key): 2*(d_c/G + d_R) flops for the score and 2*d_c/G for
    P.c_KV.  Latent rows are counted once per sequence (d_c + d_R elements).  The two
    projections are 2*T*H*d_hc*d_c/G flops each.
    """
    d_cg = cfg.d_c // cfg.groups
    elem = 2 if cfg.dtype == "bf16" else 4
    per_key = cfg.heads * (2 * (d_cg + cfg.d_R) + 2 * d_cg)
    att = 0
    kv_bytes = 0
    for L, q in zip(seq_lens, q_lens):
        L, q = int(L), int(q)
        for i in range(q):
            att += per_key * (L - q + i + 1 if cfg.causal else L)
        kv_bytes += L * (cfg.d_c + cfg.d_R) * elem
    T = int(sum(q_lens))
    proj = 2 * (2 * T * cfg.heads * cfg.d_hc * d_cg)
    w_bytes = 2 * cfg.heads * cfg.d_hc * d_cg * elem
    return att, proj, kv_bytes, w_bytes


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel, workload, splits):
    """HBM bytes per decode launch from committed rocprofv3 counters, if they were taken
    on this kernel, its current source, this workload and this split count."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel") != kernel:
        return None
    if rec.get("kernel_source_sha256_16") != source_hash(os.path.join(CSRC, KERNEL_SRC[kernel])):
        return None
    if rec.get("workload") != workload or rec.get("num_splits") != splits:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, att_flops_full, budget_s=20.0):
    """Time the fp64 oracle on a bounded sample of the same workload (whole heads of a
    prefix of the sequences) and scale to the step's algorithmic TFLOP/s."""
    import numpy as np  # noqa: F401
    import oracle.mla_oracle as om

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    B = len(w.latents)
    done_seqs = []
    t_spent = 0.0
    t0 = time.perf_counter()
    for b in range(B):
        tb = time.perf_counter()
        om.mla_decode(w.q_c, w.q_r, w.latents, w.w_uk, w.w_uv, w.cu_q, groups=w.cfg.groups,
                      rope_base=w.cfg.rope_base, causal=w.cfg.causal, seq_subset=[b])
        t_spent += time.perf_counter() - tb
        done_seqs.append(b)
        if time.perf_counter() - t0 > budget_s:
            break
    sub_lens = [w.seq_lens[b] for b in done_seqs]
    sub_q = [w.q_lens[b] for b in done_seqs]
    att, proj, _, _ = algorithmic_work(w.cfg, sub_lens, sub_q)
    tflops = (att + proj) / t_spent / 1e12
    return {
        "value": tflops, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "seqs_per_s": len(done_seqs) / t_spent,
        "sample": f"{len(done_seqs)} of {B} sequences (all heads) of {w.cfg.name}, "
                  f"fp64 non-absorbed numpy oracle, {t_spent:.1f} s",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=HEADLINE)
    ap.add_argument("--splits", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch the four calls eagerly")
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
    d = harness.to_device(w)
    step = harness.make_step(w, d, args.splits)
    S = step.num_splits
    flush_buf = None if args.no_flush else torch.ones(1 << 28, dtype=torch.float32, device="cuda")

    def flush():
        if flush_buf is not None:
            flush_buf.max()
    stream = torch.cuda.current_stream()

    def one_step(ev=None):
        if ev is None:
            step()
            return
        ev[0].record(stream)
        step.absorb()
        ev[1].record(stream)
        step.attend()
        ev[2].record(stream)
        step.merge()
        ev[3].record(stream)
        step.project()
        ev[4].record(stream)

    for _ in range(args.warmup):
        flush()
        one_step()
    torch.cuda.synchronize()

    # Per-kernel times: the four calls issued one by one with events between them
    # (the flush before each step keeps the GPU busy long enough for all four
    # launches to be queued, so the events bracket kernel execution).
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for k in range(args.steps):
        flush()
        one_step(events[k])
    torch.cuda.synchronize()
    dec_ms = [e[1].elapsed_time(e[2]) for e in events]
    parts = {name: statistics.median([e[i].elapsed_time(e[i + 1]) for e in events])
             for i, name in enumerate(["absorb_q", "decode_paged", "combine", "up_v"])}
    dec = statistics.median(dec_ms)

    # Step time: the four calls captured once as a HIP graph and replayed, so the
    # host's per-call launch cost does not sit between the kernels.
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
    ev_step = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for k in range(args.steps):
        flush()
        ev_step[k][0].record(stream)
        if graph is not None:
            graph.replay()
        else:
            step()
        ev_step[k][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = [e[0].elapsed_time(e[1]) for e in ev_step]
    ms = statistics.median(step_ms)

    att, proj, kv_bytes, w_bytes = algorithmic_work(cfg, w.seq_lens, w.q_lens)
    flops = att + proj
    tflops = flops / (ms * 1e-3) / 1e12
    kv_gbps = kv_bytes / (ms * 1e-3) / 1e9
    seqs = cfg.batch / (ms * 1e-3)

    # Dominant kernel: split-KV decode.  Bound by whichever roof is further away.
    peak_f = BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else FP32_PEAK_TFLOPS
    t_hbm = kv_bytes / (HBM_PEAK_GBPS * 1e9)
    t_mfma = att / (peak_f * 1e12)
    kernel = decode_kernel_name(cfg)
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
        "config": {"workload": cfg.name, "batch": cfg.batch, "heads": cfg.heads, "d_hc": cfg.d_hc,
                   "d_c": cfg.d_c, "d_R": cfg.d_R, "groups": cfg.groups, "page_size": cfg.page_size,
                   "seq_len": cfg.seq_len, "seq_len_range": cfg.seq_len_range,
                   "total_q": int(w.total_q), "num_splits": S,
                   "pages_per_split": step.pages_per_split, "cache_flushed": flush_buf is not None,
                   "hip_graph": graph is not None},
        "latent_kv_gbps": kv_gbps, "latent_kv_frac_hbm_peak": kv_gbps / HBM_PEAK_GBPS,
        "tflops_frac_mfma_peak": tflops / peak_f, "seqs_per_s": seqs,
        "kernel_ms": parts, "wall_s_timed_region": wall,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, att)
    print(json.dumps(out))


def decode_kernel_name(cfg):
    """The decode kernel the library dispatches for this shape (same rule as the library:
    MLA_KV_DECODE_KERNEL = generic / mfma, default the mfma kernel where it applies)."""
    mfma_shape = (cfg.dtype == "bf16" and cfg.heads == 128 and cfg.groups in (1, 2)
                  and cfg.d_c == 512 and cfg.d_R == 64 and cfg.page_size == 64)
    choice = os.environ.get("MLA_KV_DECODE_KERNEL", "")
    if choice == "generic" or not mfma_shape:
        return "decode_generic_kernel"
    return "decode_mfma_kernel"


if __name__ == "__main__":
    main()
