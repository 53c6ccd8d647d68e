"""GPU parity: the four C-ABI calls against the fp64 CPU oracle on identical seeded inputs.

Tolerance (the decode study's bar, read normwise): on the final output,
max|gpu - ref| / max|ref| <= 1e-2 and cosine similarity >= 0.99999 (float64).
Element-wise relative error is not used: outputs cross zero.
"""
import math

import numpy as np
import pytest
import torch

import oracle.mla_oracle as om
import parity_log
import spike_cases
from mla_latent_kv_09_amd import harness, mla
from mla_latent_kv_09_amd import workloads as wl

pytestmark = pytest.mark.gpu

NORM_TOL = 1e-2
COS_TOL = 0.99999


def _f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def compare(got, ref):
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    assert np.isfinite(got).all(), "non-finite values in the GPU output"
    err = np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300)
    den = np.linalg.norm(got) * np.linalg.norm(ref)
    cos = float(got @ ref / den) if den > 0 else (1.0 if np.array_equal(got, ref) else 0.0)
    return err, cos


def assert_parity(got, ref, tol=NORM_TOL, cos_tol=COS_TOL, what="out", lse_err=None, show=False):
    err, cos = compare(got, ref)
    print(f"{what}: normwise err {err:.3e}  1-cos {1 - cos:.3e}", flush=True)
    parity_log.record(what, err, cos, lse_err, tol=tol, cos_tol=cos_tol, show=show)
    assert err <= tol and cos >= cos_tol, (what, err, cos)


def oracle_for(w, *, rope=True, **kw):
    return om.mla_decode(w.q_c, w.q_r, w.latents, w.w_uk, w.w_uv, w.cu_q, groups=w.cfg.groups,
                         rope_base=w.cfg.rope_base if rope else None, causal=w.cfg.causal, **kw)


def run_step(w, *, num_splits=None, rope=True):
    d = harness.to_device(w, rope=rope)
    step = harness.make_step(w, d, num_splits)
    step()
    torch.cuda.synchronize()
    return step


def _small(name, **kw):
    return wl.CONFIGS[name].replace(**kw)


SMALL_CASES = {
    "tiny_fp32": wl.CONFIGS["tiny_fp32"],
    "dsv3_small": _small("dsv3_b16_l4096", batch=3, seq_len=300),
    "long_small": _small("long_b16_l65536", batch=2, seq_len=5000),
    "ragged_small": _small("ragged_b64", batch=6, seq_len_range=(1, 400)),
    "gla2_small": _small("gla2_b32_l16384", batch=2, seq_len=333),
}


@pytest.mark.parametrize("case", list(SMALL_CASES))
@pytest.mark.parametrize("rope", [True, False])
def test_parity_small(case, rope):
    cfg = SMALL_CASES[case]
    print(f"case {case} rope={rope}", flush=True)
    w = wl.make_workload(cfg)
    step = run_step(w, rope=rope)
    ref = oracle_for(w, rope=rope)
    fp32 = cfg.dtype == "fp32"
    lse_err = np.max(np.abs(_f64(step.lse) - ref["lse"]))
    print(f"lse max abs err {lse_err:.3e}", flush=True)
    assert_parity(_f64(step.out), ref["out"], tol=1e-4 if fp32 else NORM_TOL,
                  cos_tol=0.9999999 if fp32 else COS_TOL, lse_err=lse_err, show=rope)
    assert_parity(_f64(step.o_latent), ref["o_latent"], tol=1e-4 if fp32 else NORM_TOL,
                  cos_tol=0.9999999 if fp32 else COS_TOL, what="o_latent")
    assert lse_err <= (1e-4 if fp32 else 2e-2)


@pytest.mark.parametrize("kind", ["mfma32-128", "mfma32-64"])
@pytest.mark.parametrize("case", ["dsv3_small", "long_small", "ragged_small"])
@pytest.mark.parametrize("rope", [True, False])
def test_parity_small_mfma32(case, rope, kind, monkeypatch):
    """The 32x32x16 kernel on the one-group cases: four 32-head waves per (token, split)
    (mfma32-128), or two 64-head workgroups whose waves split each page's tokens (mfma32-64)."""
    monkeypatch.setenv("MLA_KV_DECODE_KERNEL", kind)
    cfg = SMALL_CASES[case]
    print(f"case {case} rope={rope} kernel {kind}", flush=True)
    w = wl.make_workload(cfg)
    step = run_step(w, rope=rope)
    ref = oracle_for(w, rope=rope)
    assert_parity(_f64(step.out), ref["out"])
    assert_parity(_f64(step.o_latent), ref["o_latent"], what="o_latent")
    assert np.max(np.abs(_f64(step.lse) - ref["lse"])) <= 2e-2


@pytest.mark.parametrize("batch,mix", [(1, False), (16, False), (64, True), (65, True), (70, False)])
@pytest.mark.parametrize("kind", ["mfma64", "mfma128", "mfma32-128", "mfma32-64"])
def test_batch_sizes_around_the_wave_sequence_lookup(batch, mix, kind, monkeypatch):
    """Batches of 1, 16, 64 (the largest whose sequence table one wave holds), 65 and 70
    (the binary search over cu_q), with and without two-token sequences, on every MFMA
    decode form; 16 one-token sequences with 64-head workgroups take the launch order
    that puts a token's workgroups on one XCD."""
    monkeypatch.setenv("MLA_KV_DECODE_KERNEL", kind)
    cfg = _small("ragged_b64", batch=batch, seq_len_range=(1, 160), q_len_mix=mix)
    print(f"batch {batch} q_len_mix={mix} kernel {kind}", flush=True)
    w = wl.make_workload(cfg)
    step = run_step(w, rope=True)
    ref = oracle_for(w, rope=True)
    assert_parity(_f64(step.out), ref["out"])
    assert_parity(_f64(step.o_latent), ref["o_latent"], what="o_latent")
    assert np.max(np.abs(_f64(step.lse) - ref["lse"])) <= 2e-2


@pytest.mark.parametrize("splits", [1, 3, 8, 40])
def test_split_count_invariance(splits):
    """Split count changes only rounding; empty splits (more splits than pages) are harmless."""
    w = wl.make_workload(_small("dsv3_b16_l4096", batch=2, seq_len=650))
    step = run_step(w, num_splits=splits)
    ref = oracle_for(w)
    assert_parity(_f64(step.out), ref["out"])


def test_page_permutation_invariance_bitwise():
    cfg = _small("dsv3_b16_l4096", batch=2, seq_len=777)
    a = run_step(wl.make_workload(cfg), num_splits=4)
    b = run_step(wl.make_workload(cfg.replace(identity_pages=True)), num_splits=4)
    assert torch.equal(a.out, b.out) and torch.equal(a.lse, b.lse)


def test_bitwise_repeatable():
    w = wl.make_workload(_small("ragged_b64", batch=4, seq_len_range=(60, 300)))
    d = harness.to_device(w)
    step = harness.make_step(w, d, 5)
    o1 = step().clone()
    torch.cuda.synchronize()
    o2 = step().clone()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("lens,q_lens", [
    ((1,), (1,)), ((64,), (1,)), ((65,), (1,)), ((2,), (2,)), ((128, 129, 63), (1, 2, 1)),
    ((31, 32, 33, 96, 97), (1, 1, 2, 1, 2)),
])
@pytest.mark.parametrize("heads,kind", [(16, None), (128, "mfma128"), (128, "mfma64"),
                                        (128, "mfma32-128"), (128, "mfma32-64")])
def test_edge_lengths(lens, q_lens, heads, kind, monkeypatch):
    """16 heads run the generic kernel; 128 heads the MFMA kernel with one workgroup of
    128 heads or two of 64 heads per (token, split).  Lengths of 1, 2, 31-33 and 65 keys
    leave the second token half of a split's only page, or of its last page, without a
    valid key."""
    if kind is not None:
        monkeypatch.setenv("MLA_KV_DECODE_KERNEL", kind)
    cfg = _small("dsv3_b16_l4096", batch=len(lens), seq_len=max(lens), heads=heads)
    w = _with_lengths(cfg, lens, q_lens)
    step = run_step(w, num_splits=2)
    ref = oracle_for(w)
    assert_parity(_f64(step.out), ref["out"])


def _with_lengths(cfg, lens, q_lens):
    """A workload with given per-sequence lengths and query counts (same generator streams)."""
    w = wl.make_workload(cfg.replace(seq_len=None, seq_len_range=(1, 1)))
    B = len(lens)
    rng = np.random.default_rng(1234)
    seq_lens = np.array(lens, np.int32)
    q = np.array(q_lens, np.int32)
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(q)
    T = int(cu[-1])
    rnd = wl.round_bf16
    H = cfg.heads
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
                       q_c=rnd(rng.standard_normal((T, H, cfg.d_hc)).astype(np.float32)),
                       q_r=rnd(rng.standard_normal((T, H, cfg.d_R)).astype(np.float32)),
                       latents=latents, w_uk=w.w_uk, w_uv=w.w_uv, page_table=pt, pool=pool)


@pytest.mark.parametrize("kind", ["mfma128", "mfma64", "mfma32-128", "mfma32-64", "generic"])
def test_splits_longer_than_64_pages(kind, monkeypatch):
    """One split per sequence of 70 and 140 pages (4470 and 8960 keys, the second with two
    query tokens): the MFMA kernels hold a split's page ids 64 at a time and load the next
    64 while streaming, a path no shorter split reaches."""
    monkeypatch.setenv("MLA_KV_DECODE_KERNEL", kind)
    cfg = _small("dsv3_b16_l4096", batch=2, seq_len=8960)
    w = _with_lengths(cfg, (4470, 8960), (1, 2))
    print(f"kernel {kind}: one split of 70 and of 140 pages", flush=True)
    step = run_step(w, num_splits=1)
    ref = oracle_for(w)
    assert_parity(_f64(step.out), ref["out"])
    assert np.max(np.abs(_f64(step.lse) - ref["lse"])) <= 2e-2


@pytest.mark.parametrize("heads,kind", [(16, None), (128, "mfma128"), (128, "mfma64"),
                                        (128, "mfma32-128"), (128, "mfma32-64")])
def test_empty_sequence_gives_zero_and_minus_inf(heads, kind, monkeypatch):
    """A sequence with no keys: output 0 and LSE -inf on every head, from the generic
    kernel and from both head splits of the MFMA kernel (where both workgroups of an
    empty pair leave through the early exit)."""
    if kind is not None:
        monkeypatch.setenv("MLA_KV_DECODE_KERNEL", kind)
    cfg = _small("dsv3_b16_l4096", batch=2, heads=heads, seq_len=100)
    w = wl.make_workload(cfg)
    w.seq_lens[1] = 0                       # second sequence has no keys at all
    step = run_step(w, num_splits=2)
    out = _f64(step.out)
    lse = _f64(step.lse)
    assert (out[1] == 0).all() and np.isneginf(lse[1]).all()
    ref = oracle_for(w, seq_subset=[0])
    assert_parity(out[0], ref["out"][0])


def test_non_causal_flag():
    cfg = _small("ragged_b64", batch=3, seq_len_range=(70, 200), causal=False)
    w = wl.make_workload(cfg)
    step = run_step(w)
    assert_parity(_f64(step.out), oracle_for(w)["out"])


def test_rope_table_matches_fp64():
    cos, sin = mla.rope_table(70000, 64, 10000.0)
    torch.cuda.synchronize()
    pos = np.array([0, 1, 4095, 65535, 69999])
    ang = om.rope_angles(pos, 64, 10000.0)
    assert np.max(np.abs(cos.cpu().numpy()[pos] - np.cos(ang))) <= 2 ** -24
    assert np.max(np.abs(sin.cpu().numpy()[pos] - np.sin(ang))) <= 2 ** -24


def test_zero_queries_is_a_no_op():
    cfg = _small("dsv3_b16_l4096", batch=1, heads=16, seq_len=64)
    w = wl.make_workload(cfg)
    d = harness.to_device(w)
    empty = torch.empty((0, 16, 128), dtype=torch.bfloat16, device="cuda")
    w_uk = d.w_uk
    q_abs = mla.absorb_q(empty, w_uk)
    assert q_abs.shape == (0, 16, 512)


@pytest.mark.parametrize("T", [1, 16, 37, 96])
@pytest.mark.parametrize("d_cg", [512, 256])
@pytest.mark.parametrize("d_hc", [128, 80])
def test_projections_against_reference(T, d_cg, d_hc):
    """mla_absorb_q and mla_up_v alone, on the MFMA shapes and a ragged row count.  With
    d_hc = 128 both take their LDS-staged MFMA kernels; with d_hc = 80 (not a multiple of
    64) up_v takes the one-wave-per-16-dims MFMA kernel and absorb the generic one."""
    rng = np.random.default_rng(T + d_cg + d_hc)
    H = 128
    q_c = wl.round_bf16(rng.standard_normal((T, H, d_hc)).astype(np.float32))
    w = wl.round_bf16((rng.standard_normal((H, d_hc, d_cg)) / np.sqrt(d_cg)).astype(np.float32))
    o = wl.round_bf16(rng.standard_normal((T, H, d_cg)).astype(np.float32))
    dev = lambda x: torch.from_numpy(x).to("cuda").to(torch.bfloat16)
    q_abs = mla.absorb_q(dev(q_c), dev(w))
    out = mla.up_v(dev(o), dev(w))
    torch.cuda.synchronize()
    assert_parity(_f64(q_abs), om.absorb_reference(q_c, w), what="q_abs")
    assert_parity(_f64(out), om.up_v_reference(o, w), what="up_v")


@pytest.mark.parametrize("case", ["dsv3_small", "ragged_small", "long_small", "gla2_small"])
def test_decode_kernels_agree(case, monkeypatch):
    """The decode kernels (MFMA with 128 or 64 heads per workgroup, generic) on the same
    inputs: each within tolerance of the oracle and of the generic kernel.  Three splits
    of a batch of a few tokens leave a last block of fewer than 8 (token, split) pairs
    in the head-split grid order."""
    cfg = SMALL_CASES[case]
    w = wl.make_workload(cfg)
    outs = {}
    kinds = (("mfma128", "mfma64", "mfma32-128", "mfma32-64", "generic") if cfg.groups == 1
             else ("mfma128", "generic"))
    for kind in kinds:
        monkeypatch.setenv("MLA_KV_DECODE_KERNEL", kind)
        print(f"  kernel {kind}", flush=True)
        outs[kind] = _f64(run_step(w, num_splits=3).out)
    ref = oracle_for(w)["out"]
    for kind in kinds:
        assert_parity(outs[kind], ref, what=kind)
    # Kernel against kernel: each within the bar of the oracle, with independent
    # roundings, so their difference is bounded by twice the bar.
    for kind in kinds[:-1]:
        assert_parity(outs[kind], outs["generic"], tol=2 * NORM_TOL, cos_tol=1 - 2 * (1 - COS_TOL),
                      what=f"{kind} vs generic")


@pytest.mark.parametrize("kind", ["mfma128", "mfma64", "mfma32-128", "mfma32-64", "generic"])
@pytest.mark.parametrize("case,mode", [("dsv3_small", "grow"), ("dsv3_small", "flood"),
                                       ("dsv3_small", "shrink"), ("gla2_small", "grow"),
                                       ("gla2_small", "flood")])
def test_softmax_reference_moves(kind, case, mode, monkeypatch):
    """Pages 2.. of every sequence rewritten (exactly, in bf16), one split per sequence.
    grow:   rows scaled by 4; the later pages' score maxima (std ~1.4 -> ~5.8 log2
            units) exceed the first page's by more than the kernels' softmax reference
            slack (8 log2 units) for most heads, so the running output is rescaled
            mid-split.
    flood:  every row replaced by one row scaled by 512; heads that score it positive
            see their reference jump by hundreds of log2 units (the rescale factor
            underflows to zero) and a softmax spread evenly over identical rows, so the
            output is that row exactly; the other heads keep the first pages.
    shrink: rows scaled by 1/64; the first pages keep the reference for the whole split.
    The 32x32 kernel (mfma32) moves its reference only past 2^64: grow takes later terms
    of up to about 2^17 against the first page's reference, and flood moves it.
    Scaled rows scale the rounding error of a score with them, so W_UK is a selection
    matrix (q_abs = q_c on the first d_hc latent columns, exact in bf16) and RoPE is
    off (a rotated q_R is rounded to bf16): the scores then differ from the oracle's
    by fp32 accumulation only, and the comparison tests the kernels' softmax."""
    if kind in ("mfma64", "mfma32-128", "mfma32-64") and SMALL_CASES[case].groups != 1:
        pytest.skip("the 64-head split and the 32x32 kernel exist for one latent group only")
    w = wl.make_workload(SMALL_CASES[case])
    H, d_hc, d_cg = w.w_uk.shape
    w.w_uk = np.zeros_like(w.w_uk)
    w.w_uk[:, np.arange(d_hc), np.arange(d_hc)] = 1.0
    ps = w.cfg.page_size
    for b in range(len(w.seq_lens)):
        L = int(w.seq_lens[b])
        n_pages = (L + ps - 1) // ps
        if n_pages < 3:
            continue
        first = wl.bf16_bits_to_f32(w.pool[w.page_table[b, 2], 0]).copy()
        for k in range(2, n_pages):
            pg = w.page_table[b, k]
            n = min(ps, L - k * ps)             # rows past the sequence end stay NaN
            x = wl.bf16_bits_to_f32(w.pool[pg, :n])
            if mode == "grow":
                x = x * np.float32(4.0)
            elif mode == "shrink":
                x = x * np.float32(1.0 / 64.0)
            else:
                x = np.broadcast_to(first * np.float32(512.0), x.shape)
            w.pool[pg, :n] = wl.bf16_bits(x)
    monkeypatch.setenv("MLA_KV_DECODE_KERNEL", kind)
    print(f"case {case} mode {mode} kernel {kind}", flush=True)
    step = run_step(w, num_splits=1, rope=False)
    ref = oracle_for(w, rope=False)
    assert_parity(_f64(step.o_latent), ref["o_latent"], what="o_latent")
    assert_parity(_f64(step.out), ref["out"])


@pytest.mark.parametrize("kind", ["mfma128", "mfma64", "mfma32-128", "mfma32-64", "generic"])
@pytest.mark.parametrize("slots", [(5, 9), (37, 40)])
def test_softmax_reference_moves_keep_earlier_pages(kind, slots, monkeypatch):
    """A later page moving the softmax reference must rescale what earlier pages added,
    not drop it: pages 1 and 2 carry spikes 63 and 65 log2 units above page 0's maximum
    (so only page 2 moves a reference that allows terms up to 2^64), and page 1's spike
    keeps about a fifth of the output.  Dropping it misses the bar by about 20x.  The
    spikes sit in the first or the second 32-token half of their pages."""
    cfg = wl.CONFIGS["dsv3_b16_l4096"].replace(batch=1, seq_len=4 * 64 - 7, q_len=1)
    w, gaps = spike_cases.climbing_spikes_workload(cfg, slots=slots)
    assert 62.5 < gaps[0] < 63.5 and 64.5 < gaps[1] < 65.5, gaps
    monkeypatch.setenv("MLA_KV_DECODE_KERNEL", kind)
    print(f"kernel {kind}: spikes in rows {slots} at +{gaps[0]:.2f} and +{gaps[1]:.2f} log2 units",
          flush=True)
    step = run_step(w, num_splits=1, rope=False)
    ref = oracle_for(w, rope=False)
    lat = ref["o_latent"][0, 0]
    assert 0.1 < lat[200] / lat[300] < 0.4       # the design: page 1's spike keeps weight
    assert_parity(_f64(step.o_latent), ref["o_latent"], what="o_latent")
    assert_parity(_f64(step.out), ref["out"])


@pytest.mark.parametrize("T,d_cg,S,dt", [(37, 512, 16, "bf16"), (9, 256, 70, "bf16"),
                                         (5, 512, 3, "fp32"),
                                         # more rows than resident waves: the many-row
                                         # form (several rows per wave, empty splits not read)
                                         (40, 512, 5, "bf16"), (25, 512, 17, "bf16"),
                                         (33, 512, 30, "bf16"), (40, 256, 12, "bf16"),
                                         (300, 512, 16, "fp32")])
def test_combine_against_oracle_merge(T, d_cg, S, dt):
    """mla_combine alone on synthetic partials: a third of the splits empty (LSE = -inf,
    partials NaN), one token with no keys at all, split counts past one wave's 64 lanes,
    and row counts (T x H) past the waves the chip keeps resident; o_latent and the LSE
    against the oracle's fp64 merge."""
    H = 128 if dt == "bf16" else 16
    rng = np.random.default_rng(T * 1000 + S)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    o_part = rng.standard_normal((T, H, S, d_cg)).astype(np.float32)
    if dt == "bf16":
        o_part = wl.round_bf16(o_part)
    lse = (rng.standard_normal((T, H, S)) * 3).astype(np.float32)
    empty = rng.random((T, H, S)) < 1 / 3
    empty[0] = True
    lse[empty] = -np.inf
    o_part[empty] = np.nan
    op = torch.from_numpy(o_part).to("cuda").to(tdt)
    lp = torch.from_numpy(lse).to("cuda")
    lse_out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    o_lat = mla.combine(op, lp, lse_out=lse_out, dtype=tdt)
    torch.cuda.synchronize()
    ref_o, ref_l = om.merge_splits(o_part, lse)
    assert_parity(_f64(o_lat), ref_o, tol=NORM_TOL if dt == "bf16" else 1e-6,
                  cos_tol=COS_TOL if dt == "bf16" else 0.9999999, what="o_latent")
    got_l = _f64(lse_out)
    assert np.array_equal(np.isneginf(got_l), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    assert np.max(np.abs(got_l[fin] - ref_l[fin])) < 1e-4
    assert torch.all(o_lat[0] == 0)


def test_combine_ignores_unwritten_empty_splits():
    """Empty splits leave their o_part rows unwritten; NaN there must not reach the output."""
    w = wl.make_workload(_small("ragged_b64", batch=4, seq_len_range=(10, 300)))
    d = harness.to_device(w)
    step = harness.make_step(w, d, 40)         # far more splits than pages
    step.o_part.fill_(float("nan"))
    step()
    torch.cuda.synchronize()
    assert_parity(_f64(step.out), oracle_for(w)["out"])


@pytest.mark.parametrize("case", ["dsv3_small", "gla2_small"])
def test_hip_graph_replay_matches_eager(case):
    """The four calls captured as a HIP graph: every replay equals the eager result bitwise."""
    w = wl.make_workload(SMALL_CASES[case])
    d = harness.to_device(w)
    step = harness.make_step(w, d)
    eager = step().clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for _ in range(3):
        step.out.zero_()
        torch.randn(1 << 20, device="cuda").sum()     # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out, eager)


@pytest.mark.parametrize("kind", ["mfma128", "mfma64", "mfma32-128", "mfma32-64", "generic"])
def test_split_length_of_int32_max_pages(kind, monkeypatch):
    """pages_per_split = 2^31 - 1 with two splits: the library clamps the length to the
    page table (split 0 then covers every key, split 1 none), and the kernels compute
    split bounds in 64 bits, so no key is dropped or read twice."""
    monkeypatch.setenv("MLA_KV_DECODE_KERNEL", kind)
    w = wl.make_workload(_small("ragged_b64", batch=3, seq_len_range=(100, 700)))
    d = harness.to_device(w)
    step = harness.make_step(w, d, 2, 2 ** 31 - 1)
    step()
    torch.cuda.synchronize()
    assert np.isneginf(_f64(step.lse_part)[:, :, 1]).all()
    assert_parity(_f64(step.out), oracle_for(w)["out"])
