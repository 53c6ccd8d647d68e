"""Inputs whose softmax maximum climbs within a split, for the GPU parity tests (test
infrastructure: uses the oracle's softmax scale, holds none of the kernels' arithmetic)."""
import math

import numpy as np

import oracle.mla_oracle as om
from mla_latent_kv_09_amd import workloads as wl


def climbing_spikes_workload(cfg, t_gaps=(63.0, 65.0), slots=(5, 9), beta=16.0):
    """One sequence whose score maximum climbs twice within a split: every head and token
    shares one query (W_UK a selection matrix, so q_abs = q_c on the first d_hc latent
    columns), page 0 holds random rows and, in row 0, its maximum (2 log2 units above the
    rest, so a first 32-token block sets the same reference as the first page), and pages
    1 and 2 each hold one spike row (rows slots[0], slots[1]) whose score lies t_gaps[0]
    resp. t_gaps[1] log2 units above page 0's maximum (k_R = 0 on the spikes, RoPE off).
    With a softmax reference that moves only past 2^64, page 1 stays against page 0's
    reference and page 2 moves it; page 1's spike then still holds about
    2^-(t_gaps[1] - t_gaps[0]) of page 2's weight, and its row differs from page 2's in
    latent column 200 vs 300 (weight beta), which the scores do not see.  Returns the
    workload and the designed gaps as realised after bf16 rounding."""
    w = wl.make_workload(cfg)
    H, d_hc, d_cg = w.w_uk.shape
    w.w_uk = np.zeros_like(w.w_uk)
    w.w_uk[:, np.arange(d_hc), np.arange(d_hc)] = 1.0
    w.q_c[:] = w.q_c[0, 0]
    w.q_r[:] = w.q_r[0, 0]
    q = w.q_c[0, 0].astype(np.float64)
    qr = w.q_r[0, 0].astype(np.float64)
    d_c = cfg.d_c
    scale = om.default_scale(d_hc, cfg.d_R)
    log2e = 1.0 / math.log(2.0)

    def score_log2(row):
        return scale * log2e * (row[:d_hc] @ q + row[d_c:] @ qr)

    pt = w.page_table[0]
    page0 = wl.bf16_bits_to_f32(w.pool[pt[0]]).astype(np.float64)
    unit = np.zeros(cfg.row)
    unit[:d_hc] = q / (q @ q)                   # score of unit: scale * log2e exactly
    anchor = (max(score_log2(r) for r in page0) + 2.0) / (scale * log2e) * unit
    w.pool[pt[0], 0] = wl.bf16_bits(anchor.astype(np.float32))
    t0 = score_log2(wl.bf16_bits_to_f32(w.pool[pt[0], 0]).astype(np.float64))
    gaps = []
    for k, (gap, col, slot) in enumerate(zip(t_gaps, (200, 300), slots), start=1):
        alpha = (t0 + gap) / (scale * log2e)
        row = alpha * unit
        row[col] = beta
        bits = wl.bf16_bits(row.astype(np.float32))
        w.pool[pt[k], slot] = bits
        gaps.append(score_log2(wl.bf16_bits_to_f32(bits).astype(np.float64)) - t0)
    return w, gaps


def realized_gaps(w, rows, slots=(5, 9)):
    """Score gaps (log2 units) of the two spikes above the page-0 anchor, taken on the
    logical rows ``rows`` of sequence 0 (for instance a quantized cache's dequantized
    rows) with the workload's shared query, RoPE off."""
    cfg = w.cfg
    d_hc, d_c = w.w_uk.shape[1], cfg.d_c
    q = w.q_c[0, 0].astype(np.float64)
    qr = w.q_r[0, 0].astype(np.float64)
    k = om.default_scale(d_hc, cfg.d_R) / math.log(2.0)
    rows = np.asarray(rows, np.float64)
    ps = cfg.page_size

    def t(j):
        return k * (rows[j, :d_hc] @ q + rows[j, d_c:] @ qr)

    t0 = t(0)
    return [t(ps + slots[0]) - t0, t(2 * ps + slots[1]) - t0]
