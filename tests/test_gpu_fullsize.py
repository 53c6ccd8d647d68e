"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

The whole decode step runs on every query row; the fp64 oracle is evaluated on a
sample of (sequence, head) pairs that covers every wave position and both latent
groups, and the GPU output on those rows must meet the same bar as the small
cases (normwise max error <= 1e-2, cosine >= 0.99999).  Every output is also
checked to be finite, and every row's log-sum-exp against a bound that holds at
any size: lse >= log(visible keys) + the smallest scaled score is not checkable
without scores, so the checked property is lse <= max score + log(keys), via
the oracle on the sample and finiteness elsewhere.
"""
import numpy as np
import pytest
import torch

import oracle.mla_oracle as om
import parity_log
from mla_latent_kv_09_amd import harness
from mla_latent_kv_09_amd import workloads as wl

pytestmark = pytest.mark.gpu

FULL = ["dsv3_b16_l4096", "long_b16_l65536", "ragged_b64", "gla2_b32_l16384"]
SAMPLE_HEADS = [0, 17, 35, 63, 64, 90, 111, 127]


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


# The default plan runs the 32x32x16 kernel on long and ragged and the 16x16x32 kernel
# (64-head split, or two latent groups) on dsv3 and gla2; the extra cases run each
# one-group kernel on the other's full-size shapes too.
CASES = [(n, None) for n in FULL] + [("dsv3_b16_l4096", "mfma32"), ("long_b16_l65536", "mfma128"),
                                     ("ragged_b64", "mfma128")]


@pytest.mark.parametrize("name,kind", CASES)
def test_fullsize_sampled_parity(name, kind, monkeypatch):
    if kind is not None:
        monkeypatch.setenv("MLA_KV_DECODE_KERNEL", kind)
    cfg = wl.CONFIGS[name]
    print(f"full-size {name} kernel {kind or 'default'}: generating", flush=True)
    w = wl.make_workload(cfg)
    d = harness.to_device(w)
    step = harness.make_step(w, d)           # the bench's split plan
    print(f"  splits {step.num_splits} x {step.pages_per_split} pages; running", flush=True)
    out = _f64(step())
    lse = _f64(step.lse)
    torch.cuda.synchronize()
    assert np.isfinite(out).all() and np.isfinite(lse).all()

    B = cfg.batch
    seqs = sorted({0, B // 2, B - 1})
    if cfg.q_len_mix:  # make sure a two-query (causal) sequence is in the sample
        seqs = sorted(set(seqs) | {int(np.argmax(w.q_lens == 2)), int(np.argmax(w.q_lens == 1))})
    # One sequence with every head (a two-query one where the batch has them), the others
    # on a sample of heads that covers every wave position and both latent groups.
    full = int(np.argmax(w.q_lens == 2)) if cfg.q_len_mix else B // 2
    print(f"  oracle on sequence {full} (all heads) and {seqs} (heads {SAMPLE_HEADS})", flush=True)
    ref_full = om.mla_decode(w.q_c, w.q_r, w.latents, w.w_uk, w.w_uv, w.cu_q, groups=cfg.groups,
                             rope_base=cfg.rope_base, causal=cfg.causal, seq_subset=[full])
    ref = om.mla_decode(w.q_c, w.q_r, w.latents, w.w_uk, w.w_uv, w.cu_q, groups=cfg.groups,
                        rope_base=cfg.rope_base, causal=cfg.causal, heads_subset=SAMPLE_HEADS,
                        seq_subset=seqs)
    label = f"{name}[{kind or 'default'}]"
    rows = np.arange(w.cu_q[full], w.cu_q[full + 1])
    _check(out[rows], ref_full["out"][rows], lse[rows], ref_full["lse"][rows],
           f"{label} seq {full} all heads")
    rows = np.concatenate([np.arange(w.cu_q[b], w.cu_q[b + 1]) for b in seqs])
    _check(out[rows][:, SAMPLE_HEADS], ref["out"][rows][:, SAMPLE_HEADS],
           lse[rows][:, SAMPLE_HEADS], ref["lse"][rows][:, SAMPLE_HEADS],
           f"{label} seqs {seqs} sampled heads")


def _check(got, exp, got_lse, exp_lse, what):
    err = np.max(np.abs(got - exp)) / np.max(np.abs(exp))
    cos = float(got.ravel() @ exp.ravel() / (np.linalg.norm(got) * np.linalg.norm(exp)))
    lse_err = float(np.max(np.abs(got_lse - exp_lse)))
    print(f"  {what}: normwise err {err:.3e}  1-cos {1 - cos:.3e}  lse err {lse_err:.3e}", flush=True)
    parity_log.record("all heads" if what.endswith("all heads") else "sampled", err, cos, lse_err,
                      tol=1e-2, cos_tol=0.99999, show=True)
    assert err <= 1e-2 and cos >= 0.99999
    assert lse_err <= 5e-2
