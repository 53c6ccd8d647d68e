"""GPU test of mla_attend_noalloc: decode + merge with the split partials in the
library's static device scratch, against the two existing calls (mla_decode_paged into a
caller-allocated workspace, then mla_combine) on the same inputs.  The kernels are the
same, so the results must be bitwise equal.  Two calls in a row, the second smaller, so
the second reuses the scratch the first left behind."""
import numpy as np
import pytest
import torch

from mla_latent_kv_09_amd import harness, mla
from mla_latent_kv_09_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _reference_and_noalloc(w, num_splits=None, pages_per_split=0):
    d = harness.to_device(w)
    step = harness.make_step(w, d, num_splits, pages_per_split)
    step.absorb()
    step.attend()
    step.merge()
    T, H, d_cg = step.o_latent.shape
    o_lat = torch.full((T, H, d_cg), float("nan"), dtype=step.o_latent.dtype, device="cuda")
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    mla.attend_noalloc(step.q_abs, d.q_r, d.kv, d.page_table, d.seq_lens, d.cu_q, o_lat, lse,
                       d_hc=w.cfg.d_hc, num_splits=step.num_splits, groups=w.cfg.groups,
                       rope=d.rope, causal=w.cfg.causal, pages_per_split=step.pages_per_split)
    torch.cuda.synchronize()
    return step, o_lat, lse


def test_noalloc_matches_decode_plus_combine_twice():
    big = wl.make_workload(wl.CONFIGS["dsv3_b16_l4096"])        # planner: 8 x 8 pages, 16.8 MB
    print("no-alloc call 1: dsv3_b16_l4096", flush=True)
    step, o_lat, lse = _reference_and_noalloc(big)
    assert torch.equal(o_lat, step.o_latent) and torch.equal(lse, step.lse)
    small = wl.make_workload(wl.CONFIGS["ragged_b64"].replace(batch=5, seq_len_range=(1, 700)))
    print("no-alloc call 2: ragged batch 5, 3 splits", flush=True)
    step2, o_lat2, lse2 = _reference_and_noalloc(small, num_splits=3)
    assert torch.equal(o_lat2, step2.o_latent) and torch.equal(lse2, step2.lse)
    assert np.isfinite(o_lat2.float().cpu().numpy()).all()


def test_noalloc_rejects_partials_past_the_scratch():
    w = wl.make_workload(wl.CONFIGS["dsv3_b16_l4096"].replace(batch=16, seq_len=640))
    d = harness.to_device(w)
    step = harness.make_step(w, d, 40)              # 16 x 128 x 40 x 1028 B > 64 MiB
    step.absorb()
    with pytest.raises(mla.MLAError, match="unsupported"):
        mla.attend_noalloc(step.q_abs, d.q_r, d.kv, d.page_table, d.seq_lens, d.cu_q,
                           step.o_latent, d_hc=128, num_splits=40, rope=d.rope)
