"""GPU parity of the FP8 (E4M3) latent cache: mla_append_kv_fp8 and mla_decode_paged_fp8
against the fp64 oracle (oracle/fp8_cache.py for the format and the quantizer,
oracle/mla_oracle.py for the decode over the dequantized rows).

Bars:
* append: codes and scales are integer / bit decisions taken in float32 on both sides,
  so they must match the oracle's bit for bit; the k_R part is rotated exactly as the
  bf16 append and held to that test's bound (see test_gpu_append.py); every slot the
  append does not own keeps its bytes;
* decode: the decode bar (normwise error <= 1e-2, cosine >= 0.99999) against the oracle's
  non-absorbed decode over the dequantized rows [code * scale | k_R].  Quantization
  error is not part of the comparison: both sides see the same quantized cache.
Small cases get their pages from the oracle's quantizer; the full-size cases get them
from the GPU append (whose codes are checked bit for bit below) while the oracle
quantizes its own copy of the sampled sequences.
"""
import numpy as np
import pytest
import torch

import oracle.fp8_cache as f8
import oracle.mla_oracle as om
import parity_log
import spike_cases
from mla_latent_kv_09_amd import harness, mla
from mla_latent_kv_09_amd import workloads as wl

pytestmark = pytest.mark.gpu

NORM_TOL, COS_TOL = 1e-2, 0.99999


def _small(name, **kw):
    return wl.CONFIGS[name].replace(**kw)


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _quantized(w, seqs=None):
    """Oracle codes / scales of every sequence, the FP8 pool holding them, and the
    dequantized rows the oracle decodes (None for sequences not in ``seqs``)."""
    B = len(w.seq_lens)
    codes, scales, deq = [], [], []
    for b in range(B):
        rows = np.asarray(w.latents[b])
        c, s = f8.quantize_rows(rows[:, :w.cfg.d_c])
        codes.append(c)
        scales.append(s)
        deq.append(f8.dequantized_cache_rows(rows, w.cfg.d_c) if seqs is None or b in seqs else None)
    return wl.fp8_pool(w, codes, scales), deq


def _oracle(w, deq, **kw):
    return om.mla_decode(w.q_c, w.q_r, deq, w.w_uk, w.w_uv, w.cu_q, groups=w.cfg.groups,
                         rope_base=w.cfg.rope_base, causal=w.cfg.causal, **kw)


def _check(got, ref, what, show=False, lse_err=None):
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    assert np.isfinite(got).all(), "non-finite values in the GPU output"
    err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
    cos = float(got @ ref / (np.linalg.norm(got) * np.linalg.norm(ref)))
    print(f"{what}: normwise err {err:.3e}  1-cos {1 - cos:.3e}", flush=True)
    parity_log.record(what, err, cos, lse_err, tol=NORM_TOL, cos_tol=COS_TOL, show=show)
    assert err <= NORM_TOL and cos >= COS_TOL, (what, err, cos)


def _decode(w, pool, num_splits=None, pages_per_split=0):
    d = harness.to_device(w, kv=pool)
    step = harness.make_step(w, d, num_splits, pages_per_split)
    step()
    torch.cuda.synchronize()
    return step


SMALL = {
    "dsv3_small": _small("dsv3_b16_l4096", batch=3, seq_len=300),
    "long_small": _small("long_b16_l65536", batch=2, seq_len=5000),
    "ragged_small": _small("ragged_b64", batch=6, seq_len_range=(1, 400)),
}


@pytest.mark.parametrize("kind", [None, "mfma32-128", "mfma32-64"])
@pytest.mark.parametrize("case", list(SMALL))
def test_fp8_decode_parity_small(case, kind, monkeypatch):
    if kind is not None:
        monkeypatch.setenv("MLA_KV_DECODE_KERNEL", kind)
    w = wl.make_workload(SMALL[case])
    pool, deq = _quantized(w)
    print(f"fp8 {case} kernel {kind or 'default'}", flush=True)
    step = _decode(w, pool, num_splits=3)
    ref = _oracle(w, deq)
    lse_err = float(np.max(np.abs(_f64(step.lse) - ref["lse"])))
    _check(_f64(step.out), ref["out"], "out", show=kind is None, lse_err=lse_err)
    _check(_f64(step.o_latent), ref["o_latent"], "o_latent")
    assert lse_err <= 2e-2


@pytest.mark.parametrize("kind", ["mfma32-128", "mfma32-64"])
@pytest.mark.parametrize("slots", [(5, 9), (37, 40)])
def test_fp8_reference_moves_keep_earlier_pages(kind, slots, monkeypatch):
    """The FP8 decode's softmax on a score maximum that climbs twice within a split (the
    bf16 decode's spike case, quantized): page 2's reference move must rescale page 1's
    spike.  The gaps are checked on the dequantized rows the oracle decodes."""
    cfg = _small("dsv3_b16_l4096", batch=1, seq_len=4 * 64 - 7, q_len=1)
    w, _ = spike_cases.climbing_spikes_workload(cfg, slots=slots)
    pool, deq = _quantized(w)
    gaps = spike_cases.realized_gaps(w, deq[0], slots)
    assert 62.0 < gaps[0] < 64.0 and 64.0 < gaps[1] < 66.0, gaps
    monkeypatch.setenv("MLA_KV_DECODE_KERNEL", kind)
    print(f"fp8 kernel {kind}: spikes in rows {slots} at +{gaps[0]:.2f} and +{gaps[1]:.2f}", flush=True)
    d = harness.to_device(w, rope=False, kv=pool)
    step = harness.make_step(w, d, 1)
    step()
    torch.cuda.synchronize()
    ref = om.mla_decode(w.q_c, w.q_r, deq, w.w_uk, w.w_uv, w.cu_q, rope_base=None, causal=w.cfg.causal)
    _check(_f64(step.o_latent), ref["o_latent"], "o_latent")
    _check(_f64(step.out), ref["out"], "out")


def _with_lengths(cfg, lens, q_lens):
    """A bf16 workload with given per-sequence lengths and query counts."""
    w = wl.make_workload(cfg.replace(seq_len=None, seq_len_range=(1, 1)))
    B = len(lens)
    rng = np.random.default_rng(4321)
    seq_lens = np.array(lens, np.int32)
    q = np.array(q_lens, np.int32)
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(q)
    T = int(cu[-1])
    rnd = wl.round_bf16
    latents = [rnd(rng.standard_normal((L, cfg.row)).astype(np.float32)) for L in lens]
    n_pages = [(L + 63) // 64 for L in lens]
    P = sum(n_pages)
    perm = rng.permutation(P)
    pt = np.full((B, max(n_pages)), -1, np.int32)
    pool = np.full((P, 64, cfg.row), wl.BF16_NAN_BITS, np.uint16)
    off = 0
    for b, L in enumerate(lens):
        bits = wl.bf16_bits(latents[b])
        for k in range(n_pages[b]):
            pt[b, k] = perm[off + k]
            ch = bits[k * 64:(k + 1) * 64]
            pool[perm[off + k], :ch.shape[0]] = ch
        off += n_pages[b]
    return wl.Workload(cfg=cfg, seq_lens=seq_lens, q_lens=q, cu_q=cu,
                       q_c=rnd(rng.standard_normal((T, cfg.heads, cfg.d_hc)).astype(np.float32)),
                       q_r=rnd(rng.standard_normal((T, cfg.heads, cfg.d_R)).astype(np.float32)),
                       latents=latents, w_uk=w.w_uk, w_uv=w.w_uv, page_table=pt, pool=pool)


@pytest.mark.parametrize("lens,q_lens,splits", [
    ((1,), (1,), 1), ((64,), (1,), 1), ((65,), (1,), 1), ((2,), (2,), 1),
    ((128, 129, 63), (1, 2, 1), 2), ((31, 32, 33, 96, 97), (1, 1, 2, 1, 2), 2),
    ((130, 200), (1, 2), 1),                 # three and four pages: the copies run two ahead
    ((4470, 8960), (1, 2), 1),               # 70 and 140 pages: page ids read 64 at a time
])
@pytest.mark.parametrize("kind", ["mfma32-128", "mfma32-64"])
def test_fp8_edge_lengths(lens, q_lens, splits, kind, monkeypatch):
    """Partial pages (NaN codes, NaN k_R and NaN scales in the slots past the end),
    splits of one to 140 pages, and both head splits."""
    monkeypatch.setenv("MLA_KV_DECODE_KERNEL", kind)
    cfg = _small("dsv3_b16_l4096", batch=len(lens), seq_len=max(lens))
    w = _with_lengths(cfg, lens, q_lens)
    pool, deq = _quantized(w)
    step = _decode(w, pool, num_splits=splits)
    _check(_f64(step.out), _oracle(w, deq)["out"], f"{kind} {lens}")


def _pool_parts(pool, P, d_c, d_R):
    ps = 64
    codes = pool[:, : ps * d_c].reshape(P, ps, d_c)
    rope = pool[:, ps * d_c: ps * (d_c + 2 * d_R)].view(np.uint16).reshape(P, ps, d_R)
    scales = pool[:, ps * (d_c + 2 * d_R):].view(np.float32).reshape(P, ps)
    return codes, rope, scales


@pytest.mark.parametrize("rope", [True, False])
@pytest.mark.parametrize("case", ["dsv3_small", "ragged_small"])
def test_fp8_append_matches_oracle(case, rope):
    """The step's new tokens appended into an FP8 pool: codes and scales bit for bit
    against the oracle's quantizer, k_R within the bf16 append's bound, every other
    byte untouched."""
    w = wl.make_workload(SMALL[case])
    new = wl.make_new_tokens(w)
    pool, _ = _quantized(w)
    d = harness.to_device(w, kv=pool, rope=rope)
    c = harness._storage_tensor(w, new.c_kv, d.kv.device)
    k = harness._storage_tensor(w, new.k_r, d.kv.device)
    mla.append_kv_fp8(c, k, d.kv, d.page_table, d.seq_lens, d.cu_q, rope=d.rope if rope else None)
    torch.cuda.synchronize()
    got = d.kv.cpu().numpy()
    cfg = w.cfg
    P = w.num_pool_pages
    g_codes, g_rope, g_scales = _pool_parts(got, P, cfg.d_c, cfg.d_R)
    want_codes, want_scales = f8.quantize_rows(new.c_kv)
    exact = om.append_rows(new.c_kv, new.k_r, w.seq_lens, w.cu_q, cfg.rope_base if rope else None)
    pos = om.new_token_positions(w.seq_lens, w.cu_q)
    owned = np.zeros(got.shape, bool)   # bytes of the pages the append writes
    d_c, d_R = cfg.d_c, cfg.d_R
    for b in range(cfg.batch):
        for t in range(int(w.cu_q[b]), int(w.cu_q[b + 1])):
            p = int(pos[t])
            page, slot = int(w.page_table[b, p // 64]), p % 64
            assert np.array_equal(g_codes[page, slot], want_codes[t]), (t, "codes")
            assert g_scales[page, slot].view(np.uint32) == want_scales[t].view(np.uint32), (t, "scale")
            y = wl.bf16_bits_to_f32(g_rope[page, slot]).astype(np.float64)
            x = np.asarray(new.k_r[t], np.float64)
            e32 = 4 * 2.0 ** -24 * np.repeat(np.abs(x[0::2]) + np.abs(x[1::2]), 2)
            y_ex = exact[t, cfg.d_c:]
            assert np.all(np.abs(y - y_ex) <= e32 + 2.0 ** -8 * (np.abs(y_ex) + e32)), (t, "k_R")
            owned[page, slot * d_c:(slot + 1) * d_c] = True
            owned[page, 64 * d_c + 2 * d_R * slot:64 * d_c + 2 * d_R * (slot + 1)] = True
            owned[page, 64 * (d_c + 2 * d_R) + 4 * slot:64 * (d_c + 2 * d_R) + 4 * (slot + 1)] = True
    assert np.array_equal(got[~owned], pool[~owned])


def test_fp8_bulk_append_equals_oracle_quantizer():
    """Whole sequences appended from position 0 (the bench's way of filling an FP8 cache):
    every slot of every sequence bit for bit equal to the pages built from the oracle's
    quantizer."""
    w = wl.make_workload(_small("ragged_b64", batch=8, seq_len_range=(1, 900)))
    d = harness.to_device(w)
    got = harness.fp8_pool_by_append(w, d).cpu().numpy()
    want, _ = _quantized(w)
    cfg = w.cfg
    P = w.num_pool_pages
    g = _pool_parts(got, P, cfg.d_c, cfg.d_R)
    e = _pool_parts(want, P, cfg.d_c, cfg.d_R)
    for b in range(cfg.batch):
        L = int(w.seq_lens[b])
        for k in range((L + 63) // 64):
            pg, n = int(w.page_table[b, k]), min(64, L - 64 * k)
            for part_g, part_e in zip(g, e):
                assert np.array_equal(part_g[pg, :n].view(np.uint8), part_e[pg, :n].view(np.uint8)), (b, k)


FULL_SAMPLE_HEADS = [0, 17, 35, 63, 64, 90, 111, 127]


@pytest.mark.parametrize("name", ["dsv3_b16_l4096", "long_b16_l65536", "ragged_b64"])
def test_fp8_fullsize_sampled_parity(name):
    """The full workloads in the bench's launch configuration (the planner's splits), the
    FP8 pages written by the GPU append; one sequence on every head, three on a sample."""
    cfg = wl.CONFIGS[name]
    print(f"fp8 full-size {name}: generating", flush=True)
    w = wl.make_workload(cfg)
    d = harness.to_device(w)
    kv8 = harness.fp8_pool_by_append(w, d)
    d.kv = kv8
    step = harness.make_step(w, d)
    print(f"  splits {step.num_splits} x {step.pages_per_split} pages; running", flush=True)
    out = _f64(step())
    lse = _f64(step.lse)
    torch.cuda.synchronize()
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    B = cfg.batch
    full = int(np.argmax(w.q_lens == 2)) if cfg.q_len_mix else B // 2
    # the long sequences (65536 keys) cost the CPU quantizer about 20 s each: two of them
    seqs = sorted({B - 1, full} if cfg.seq_len and cfg.seq_len > 32768 else {0, B // 2, B - 1, full})
    deq = [f8.dequantized_cache_rows(np.asarray(w.latents[b]), cfg.d_c) if b in seqs else None
           for b in range(B)]
    ref_full = _oracle(w, deq, seq_subset=[full])
    rows = np.arange(w.cu_q[full], w.cu_q[full + 1])
    _check(out[rows], ref_full["out"][rows], "all heads", show=True,
           lse_err=float(np.max(np.abs(lse[rows] - ref_full["lse"][rows]))))
    rest = [b for b in seqs if b != full]
    ref = _oracle(w, deq, seq_subset=rest, heads_subset=FULL_SAMPLE_HEADS)
    rows = np.concatenate([np.arange(w.cu_q[b], w.cu_q[b + 1]) for b in rest])
    _check(out[rows][:, FULL_SAMPLE_HEADS], ref["out"][rows][:, FULL_SAMPLE_HEADS], "sampled",
           show=True)
