"""GPU parity of the decompressed branch (mla_prefill_paged) and of the threshold dispatch
against the fp64 oracle.

* The K / V workspace the branch writes (W_UK c_j and W_UV c_j per head, fp32 accumulation
  rounded once to bf16) against the oracle's reconstruct_kv: normwise <= 1e-2 and
  cosine >= 0.99999 over every written row, the same bar as the decode.
* The branch's output against the oracle's non-absorbed decode (which is exactly this
  branch's definition): the decode bar, on prompts (q_len = L), prompts with history
  (q_len < L), query blocks with a ragged tail, RoPE on and off, causal and not.
* The dispatch: a batch whose largest query count reaches the threshold takes this
  branch, one below it the four absorbed calls; both meet the bar on the same inputs.
"""
import numpy as np
import pytest
import torch

import oracle.mla_oracle as om
import parity_log
import spike_cases
from mla_latent_kv_09_amd import harness, mla
from mla_latent_kv_09_amd import workloads as wl

pytestmark = pytest.mark.gpu

NORM_TOL, COS_TOL = 1e-2, 0.99999


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check(got, ref, what, show=False, lse_err=None, tol=NORM_TOL, cos_tol=COS_TOL):
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    assert np.isfinite(got).all(), "non-finite values in the GPU output"
    err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
    cos = float(got @ ref / (np.linalg.norm(got) * np.linalg.norm(ref)))
    print(f"{what}: normwise err {err:.3e}  1-cos {1 - cos:.3e}", flush=True)
    parity_log.record(what, err, cos, lse_err, tol=tol, cos_tol=cos_tol, show=show)
    assert err <= tol and cos >= cos_tol, (what, err, cos)


def _prefill_cfg(batch, q_len, seq_len, heads=128, **kw):
    return wl.CONFIGS["dsv3_b16_l4096"].replace(name="prefill_case", batch=batch, q_len=q_len,
                                                seq_len=seq_len, heads=heads, **kw)


def _run(w, *, rope=True, threshold=mla.PREFILL_THRESHOLD):
    d = harness.to_device(w, rope=rope)
    step = harness.make_step(w, d, threshold=threshold)
    step()
    torch.cuda.synchronize()
    return step, d


def _oracle(w, rope=True, **kw):
    return om.mla_decode(w.q_c, w.q_r, w.latents, w.w_uk, w.w_uv, w.cu_q, groups=w.cfg.groups,
                         rope_base=w.cfg.rope_base if rope else None, causal=w.cfg.causal, **kw)


@pytest.mark.parametrize("batch,q_len,seq_len,heads", [
    (2, 300, 700, 128),      # prompts with history, a ragged last query block
    (1, 257, 257, 128),      # a whole prompt, one query past two blocks of 128
    (3, 256, 256, 16),       # exactly the threshold, 16 heads
    (2, 400, 450, 32),
])
@pytest.mark.parametrize("rope", [True, False])
def test_prefill_matches_oracle(batch, q_len, seq_len, heads, rope):
    w = wl.make_workload(_prefill_cfg(batch, q_len, seq_len, heads))
    print(f"prefill B={batch} q={q_len} L={seq_len} H={heads} rope={rope}", flush=True)
    step, _ = _run(w, rope=rope)
    assert step.branch == mla.BRANCH_DECOMPRESSED
    ref = _oracle(w, rope=rope)
    lse_err = float(np.max(np.abs(_f64(step.lse) - ref["lse"])))
    _check(_f64(step.out), ref["out"], f"q{q_len} L{seq_len}", show=rope and heads == 128,
           lse_err=lse_err)
    assert lse_err <= 2e-2


@pytest.mark.parametrize("slots", [(5, 9), (37, 40)])
def test_prefill_reference_moves_keep_earlier_pages(slots):
    """The decompressed branch's softmax on a score maximum that climbs twice within the
    keys every query sees (pages 1 and 2 hold spikes 63 and 65 log2 units above page 0's
    maximum, one shared query): the move at page 2 must rescale page 1's spike, which
    keeps about a fifth of the weight (dropping it misses the bar about 6x)."""
    w, gaps = spike_cases.climbing_spikes_workload(_prefill_cfg(1, 256, 448), slots=slots)
    assert 62.5 < gaps[0] < 63.5 and 64.5 < gaps[1] < 65.5, gaps
    print(f"prefill spikes in rows {slots} at +{gaps[0]:.2f} and +{gaps[1]:.2f} log2 units", flush=True)
    step, _ = _run(w, rope=False)
    assert step.branch == mla.BRANCH_DECOMPRESSED
    _check(_f64(step.out), _oracle(w, rope=False)["out"], f"climbing spikes {slots}")


def test_prefill_workspace_holds_the_reconstructed_keys_and_values():
    w = wl.make_workload(_prefill_cfg(2, 260, 330))
    step, d = _run(w)
    cfg = w.cfg
    H, P = cfg.heads, w.num_pool_pages
    ws = step.workspace.view(torch.bfloat16).float().cpu().numpy()
    half = P * 64 * H * cfg.d_hc
    k_ws = ws[:half].reshape(P * 64, H, cfg.d_hc)
    v_ws = ws[half:2 * half].reshape(P * 64, H, cfg.d_hc)
    for b in range(cfg.batch):
        rows = np.asarray(w.latents[b])
        L = rows.shape[0]
        k_ref, v_ref = om.reconstruct_kv(rows[:, :cfg.d_c], w.w_uk, w.w_uv)
        phys = w.page_table[b, np.arange(L) // 64].astype(np.int64) * 64 + np.arange(L) % 64
        _check(k_ws[phys], k_ref, f"K seq {b}")
        _check(v_ws[phys], v_ref, f"V seq {b}")


def test_prefill_without_causal_mask():
    w = wl.make_workload(_prefill_cfg(2, 270, 400, causal=False))
    step, _ = _run(w)
    _check(_f64(step.out), _oracle(w)["out"], "non-causal")


def test_prefill_batch_with_short_sequences():
    """Unequal lengths and query counts in one decompressed batch: a long prompt next to
    sequences of 1-3 queries and keys short of one page (pages past their end are NaN)."""
    cfg = wl.CONFIGS["ragged_b64"].replace(batch=4, seq_len_range=(1, 1), q_len_mix=False)
    w = wl.make_workload(cfg)
    rng = np.random.default_rng(11)
    lens, q_lens = [600, 40, 3, 130], [300, 2, 3, 1]
    w2 = _with_lengths(w, lens, q_lens, rng)
    step, _ = _run(w2)
    assert step.branch == mla.BRANCH_DECOMPRESSED
    _check(_f64(step.out), _oracle(w2)["out"], "mixed lengths")


def _with_lengths(w, lens, q_lens, rng):
    cfg = w.cfg
    B = len(lens)
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


@pytest.mark.parametrize("q_len", [255, 256])
def test_dispatch_at_the_threshold_and_both_branches_agree(q_len):
    """q_len 255 takes the absorbed calls, 256 the decompressed branch; on the same inputs
    each meets the bar against the oracle and against the other branch."""
    w = wl.make_workload(_prefill_cfg(2, q_len, 500))
    d = harness.to_device(w)
    auto = harness.make_step(w, d, threshold=mla.PREFILL_THRESHOLD)
    assert auto.branch == (mla.BRANCH_DECOMPRESSED if q_len >= 256 else mla.BRANCH_ABSORBED)
    absorbed = harness.make_step(w, d)             # no threshold: always absorbed
    dec = harness.make_step(w, d, threshold=1)     # any prompt: decompressed
    out_auto = _f64(auto())
    out_abs = _f64(absorbed())
    out_dec = _f64(dec())
    torch.cuda.synchronize()
    ref = _oracle(w)["out"]
    _check(out_auto, ref, f"dispatch q{q_len}")
    _check(out_abs, ref, "absorbed")
    _check(out_dec, ref, "decompressed")
    # Two bf16 paths, each within the bar of the oracle with independent roundings: their
    # difference is bounded by the sum, twice the bar (measured 1 - cos about 9e-6).
    _check(out_dec, out_abs, "decompressed vs absorbed", tol=2 * NORM_TOL, cos_tol=1 - 2 * (1 - COS_TOL))


def test_prefill_fullsize_sampled():
    """The page's dispatch workload (batch 8, 4096-token prompts), bench launch
    configuration; the oracle on every query of one sequence for a sample of heads."""
    cfg = wl.CONFIGS["prefill_b8_l4096"]
    print("prefill full size: generating", flush=True)
    w = wl.make_workload(cfg)
    step, _ = _run(w)
    out = _f64(step.out)
    assert np.isfinite(out).all()
    heads = [0, 45, 90, 127]
    print(f"  oracle on sequence 3, heads {heads}", flush=True)
    ref = _oracle(w, heads_subset=heads, seq_subset=[3])
    rows = np.arange(w.cu_q[3], w.cu_q[4])
    _check(out[rows][:, heads], ref["out"][rows][:, heads], "all queries", show=True,
           lse_err=float(np.max(np.abs(_f64(step.lse)[rows][:, heads] - ref["lse"][rows][:, heads]))))
