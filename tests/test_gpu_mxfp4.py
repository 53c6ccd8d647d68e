"""GPU parity of the MXFP4 latent cache: mla_append_kv_mxfp4 and mla_decode_paged_mxfp4
against the fp64 oracle (oracle/mxfp4_cache.py for the format and the quantizer,
oracle/mla_oracle.py for the decode over the dequantized rows).

Bars:
* append: codes and scale bytes are integer decisions taken on exact values on both sides
  (x * 2^-e is exact in float32 and float64), so they must match the oracle's bit for
  bit; the k_R part is rotated exactly as the bf16 append and held to that test's bound;
  every byte the append does not own keeps its value;
* decode: the decode bar (normwise error <= 1e-2, cosine >= 0.99999) against the oracle's
  non-absorbed decode over the dequantized rows [E2M1(code) * 2^e | k_R].  Quantization
  error is not part of the comparison: both sides see the same quantized cache.
Small cases get their pages from the oracle's quantizer; the full-size cases get them
from the GPU append (whose codes are checked bit for bit below) while the oracle
quantizes its own copy of the sampled sequences.
"""
import numpy as np
import pytest
import torch

import oracle.mla_oracle as om
import oracle.mxfp4_cache as f4
import parity_log
import spike_cases
from mla_latent_kv_09_amd import harness, mla
from mla_latent_kv_09_amd import workloads as wl
from test_gpu_fp8 import _with_lengths

pytestmark = pytest.mark.gpu

NORM_TOL, COS_TOL = 1e-2, 0.99999


def _small(name, **kw):
    return wl.CONFIGS[name].replace(**kw)


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _quantized(w, seqs=None):
    """Oracle codes / scales of every sequence, the MXFP4 pool holding them, and the
    dequantized rows the oracle decodes (None for sequences not in ``seqs``)."""
    B = len(w.seq_lens)
    packed, scales, deq = [], [], []
    for b in range(B):
        rows = np.asarray(w.latents[b])
        p, s = f4.quantize_rows(rows[:, :w.cfg.d_c])
        packed.append(p)
        scales.append(s)
        deq.append(f4.dequantized_cache_rows(rows, w.cfg.d_c) if seqs is None or b in seqs else None)
    return wl.mxfp4_pool(w, packed, scales), deq


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


def test_page_bytes_and_format_detection():
    assert mla.mxfp4_page_bytes(512, 64) == 64 * (256 + 128 + 16) == 25600
    kv = torch.empty((3, 25600), dtype=torch.uint8, device="cuda")
    assert mla.cache_format(kv, 512, 64) == "mxfp4"
    kv8 = torch.empty((3, mla.fp8_page_bytes(512, 64)), dtype=torch.uint8, device="cuda")
    assert mla.cache_format(kv8, 512, 64) == "fp8"


@pytest.mark.parametrize("kind", [None, "mfma32-128", "mfma32-64"])
@pytest.mark.parametrize("case", list(SMALL))
def test_mxfp4_decode_parity_small(case, kind, monkeypatch):
    if kind is not None:
        monkeypatch.setenv("MLA_KV_DECODE_KERNEL", kind)
    w = wl.make_workload(SMALL[case])
    pool, deq = _quantized(w)
    print(f"mxfp4 {case} kernel {kind or 'default'}", flush=True)
    step = _decode(w, pool, num_splits=3)
    ref = _oracle(w, deq)
    lse_err = float(np.max(np.abs(_f64(step.lse) - ref["lse"])))
    _check(_f64(step.out), ref["out"], "out", show=kind is None, lse_err=lse_err)
    _check(_f64(step.o_latent), ref["o_latent"], "o_latent")
    assert lse_err <= 2e-2


@pytest.mark.parametrize("kind", ["mfma32-128", "mfma32-64"])
@pytest.mark.parametrize("slots", [(5, 9), (37, 40)])
def test_mxfp4_reference_moves_keep_earlier_pages(kind, slots, monkeypatch):
    """The bf16 decode's spike case over an MXFP4 cache: a score maximum that climbs twice
    within a split; page 2's reference move must rescale page 1's spike.  The gaps are
    checked on the dequantized rows the oracle decodes."""
    cfg = _small("dsv3_b16_l4096", batch=1, seq_len=4 * 64 - 7, q_len=1)
    w, _ = spike_cases.climbing_spikes_workload(cfg, slots=slots)
    pool, deq = _quantized(w)
    gaps = spike_cases.realized_gaps(w, deq[0], slots)
    assert 62.0 < gaps[0] < 64.0 and 64.0 < gaps[1] < 66.0, gaps
    monkeypatch.setenv("MLA_KV_DECODE_KERNEL", kind)
    print(f"mxfp4 kernel {kind}: spikes in rows {slots} at +{gaps[0]:.2f} and +{gaps[1]:.2f}", flush=True)
    d = harness.to_device(w, rope=False, kv=pool)
    step = harness.make_step(w, d, 1)
    step()
    torch.cuda.synchronize()
    ref = om.mla_decode(w.q_c, w.q_r, deq, w.w_uk, w.w_uv, w.cu_q, rope_base=None, causal=w.cfg.causal)
    _check(_f64(step.o_latent), ref["o_latent"], "o_latent")
    _check(_f64(step.out), ref["out"], "out")


@pytest.mark.parametrize("lens,q_lens,splits", [
    ((1,), (1,), 1), ((64,), (1,), 1), ((65,), (1,), 1), ((2,), (2,), 1),
    ((128, 129, 63), (1, 2, 1), 2), ((31, 32, 33, 96, 97), (1, 1, 2, 1, 2), 2),
    ((130, 200), (1, 2), 1),
    ((4470, 8960), (1, 2), 1),               # 70 and 140 pages: page ids read 64 at a time
])
@pytest.mark.parametrize("kind", ["mfma32-128", "mfma32-64"])
def test_mxfp4_edge_lengths(lens, q_lens, splits, kind, monkeypatch):
    """Partial pages (0xFF codes, NaN k_R and out-of-format scale bytes in the slots past
    the end), splits of one to 140 pages, and both head splits."""
    monkeypatch.setenv("MLA_KV_DECODE_KERNEL", kind)
    cfg = _small("dsv3_b16_l4096", batch=len(lens), seq_len=max(lens))
    w = _with_lengths(cfg, lens, q_lens)
    pool, deq = _quantized(w)
    step = _decode(w, pool, num_splits=splits)
    _check(_f64(step.out), _oracle(w, deq)["out"], f"mxfp4 {kind} {lens}")


def _pool_parts(pool, P, d_c, d_R):
    ps, cb, sb = 64, d_c // 2, d_c // 32
    codes = pool[:, : ps * cb].reshape(P, ps, cb)
    rope = pool[:, ps * cb: ps * (cb + 2 * d_R)].view(np.uint16).reshape(P, ps, d_R)
    scales = pool[:, ps * (cb + 2 * d_R):].reshape(P, ps, sb)
    return codes, rope, scales


@pytest.mark.parametrize("rope", [True, False])
@pytest.mark.parametrize("case", ["dsv3_small", "ragged_small"])
def test_mxfp4_append_matches_oracle(case, rope):
    """The step's new tokens appended into an MXFP4 pool: codes and scale bytes bit for
    bit against the oracle's quantizer, k_R within the bf16 append's bound, every other
    byte untouched."""
    w = wl.make_workload(SMALL[case])
    new = wl.make_new_tokens(w)
    pool, _ = _quantized(w)
    d = harness.to_device(w, kv=pool, rope=rope)
    c = harness._storage_tensor(w, new.c_kv, d.kv.device)
    k = harness._storage_tensor(w, new.k_r, d.kv.device)
    mla.append_kv_mxfp4(c, k, d.kv, d.page_table, d.seq_lens, d.cu_q, rope=d.rope if rope else None)
    torch.cuda.synchronize()
    got = d.kv.cpu().numpy()
    cfg = w.cfg
    P = w.num_pool_pages
    g_codes, g_rope, g_scales = _pool_parts(got, P, cfg.d_c, cfg.d_R)
    want_codes, want_scales = f4.quantize_rows(new.c_kv)
    exact = om.append_rows(new.c_kv, new.k_r, w.seq_lens, w.cu_q, cfg.rope_base if rope else None)
    pos = om.new_token_positions(w.seq_lens, w.cu_q)
    owned = np.zeros(got.shape, bool)   # bytes of the pages the append writes
    cb, sb, d_R = cfg.d_c // 2, cfg.d_c // 32, cfg.d_R
    for b in range(cfg.batch):
        for t in range(int(w.cu_q[b]), int(w.cu_q[b + 1])):
            p = int(pos[t])
            page, slot = int(w.page_table[b, p // 64]), p % 64
            assert np.array_equal(g_codes[page, slot], want_codes[t]), (t, "codes")
            assert np.array_equal(g_scales[page, slot], want_scales[t]), (t, "scales")
            y = wl.bf16_bits_to_f32(g_rope[page, slot]).astype(np.float64)
            x = np.asarray(new.k_r[t], np.float64)
            e32 = 4 * 2.0 ** -24 * np.repeat(np.abs(x[0::2]) + np.abs(x[1::2]), 2)
            y_ex = exact[t, cfg.d_c:]
            assert np.all(np.abs(y - y_ex) <= e32 + 2.0 ** -8 * (np.abs(y_ex) + e32)), (t, "k_R")
            owned[page, slot * cb:(slot + 1) * cb] = True
            owned[page, 64 * cb + 2 * d_R * slot:64 * cb + 2 * d_R * (slot + 1)] = True
            owned[page, 64 * (cb + 2 * d_R) + sb * slot:64 * (cb + 2 * d_R) + sb * (slot + 1)] = True
    assert np.array_equal(got[~owned], pool[~owned])


def test_mxfp4_append_of_extreme_blocks():
    """Blocks the quantizer clamps or saturates: all zero, far below the smallest scale,
    negative zeros, a maximum just below a power of two, ties of every E2M1 midpoint and
    values past the saturation point; codes and scale bytes bit for bit."""
    cfg = _small("dsv3_b16_l4096", batch=1, seq_len=8, q_len=8)
    w = _with_lengths(cfg, (8,), (8,))
    rows = np.zeros((8, cfg.d_c), np.float32)
    rows[1, :] = 2.0 ** -130                                   # bf16 subnormal: clamped scale
    rows[2, :] = -0.0
    rows[3, :32] = np.linspace(-7.99, 7.99, 32)                # maximum just below 8
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    rows[4, :32] = np.concatenate([mids, -mids, mids / 2, mids * 2])   # amax 12 -> e = 1
    rows[5, :] = np.tile(np.array([1e30, -1e30, 3.0, 0.0], np.float32), cfg.d_c // 4)
    rows[6, :] = wl.round_bf16(np.random.default_rng(9).standard_normal(cfg.d_c).astype(np.float32) * 1e-20)
    rows[7, :] = wl.round_bf16(np.random.default_rng(10).standard_normal(cfg.d_c).astype(np.float32) * 1e20)
    rows = wl.round_bf16(rows)
    k_r = np.zeros((8, cfg.d_R), np.float32)
    d = harness.to_device(w)
    pool = torch.zeros((w.num_pool_pages, mla.mxfp4_page_bytes(cfg.d_c, cfg.d_R)), dtype=torch.uint8,
                       device="cuda")
    c = harness._storage_tensor(w, rows, d.kv.device)
    k = harness._storage_tensor(w, k_r, d.kv.device)
    seq_lens = torch.tensor([8], dtype=torch.int32, device="cuda")
    cu = torch.tensor([0, 8], dtype=torch.int32, device="cuda")
    mla.append_kv_mxfp4(c, k, pool, d.page_table, seq_lens, cu)
    torch.cuda.synchronize()
    codes, _, scales = _pool_parts(pool.cpu().numpy(), w.num_pool_pages, cfg.d_c, cfg.d_R)
    pg = int(w.page_table[0, 0])
    want_c, want_s = f4.quantize_rows(rows)
    assert np.array_equal(scales[pg, :8], want_s)
    assert np.array_equal(codes[pg, :8], want_c)
    assert list(want_s[1]) == [1] * 16 and np.all(f4.unpack_codes(want_c[2]) == 8)


def test_mxfp4_bulk_append_equals_oracle_quantizer():
    """Whole sequences appended from position 0 (the bench's way of filling an MXFP4
    cache): every slot of every sequence bit for bit equal to the pages built from the
    oracle's quantizer."""
    w = wl.make_workload(_small("ragged_b64", batch=8, seq_len_range=(1, 900)))
    d = harness.to_device(w)
    got = harness.quant_pool_by_append(w, d, "mxfp4").cpu().numpy()
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
def test_mxfp4_fullsize_sampled_parity(name):
    """The full workloads in the bench's launch configuration (the planner's splits), the
    MXFP4 pages written by the GPU append; one sequence on every head, more on a sample."""
    cfg = wl.CONFIGS[name]
    print(f"mxfp4 full-size {name}: generating", flush=True)
    w = wl.make_workload(cfg)
    d = harness.to_device(w)
    d.kv = harness.quant_pool_by_append(w, d, "mxfp4")
    step = harness.make_step(w, d)
    print(f"  splits {step.num_splits} x {step.pages_per_split} pages; running", flush=True)
    out = _f64(step())
    lse = _f64(step.lse)
    torch.cuda.synchronize()
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    B = cfg.batch
    full = int(np.argmax(w.q_lens == 2)) if cfg.q_len_mix else B // 2
    seqs = sorted({B - 1, full} if cfg.seq_len and cfg.seq_len > 32768 else {0, B // 2, B - 1, full})
    deq = [f4.dequantized_cache_rows(np.asarray(w.latents[b]), cfg.d_c) if b in seqs else None
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
