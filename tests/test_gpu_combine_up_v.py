"""GPU tests of mla_combine_up_v: the split merge and the value up-projection as one call.

Where its fused kernel covers the shape the call must reproduce mla_combine followed by
mla_up_v bit for bit (out, o_latent, lse_out), with or without o_latent; elsewhere it
runs those two calls.  Against the fp64 oracle (merge of the splits by their LSE, then
W_UV) it holds the decode study's normwise bar like the two calls.
"""
import numpy as np
import pytest
import torch

import oracle.mla_oracle as om
import parity_log
from mla_latent_kv_09_amd import mla
from mla_latent_kv_09_amd import workloads as wl

pytestmark = pytest.mark.gpu

NORM_TOL = 1e-2
COS_TOL = 0.99999


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _partials(T, H, S, d_cg, d_hc, seed):
    """Split partials with a third of the splits empty (LSE = -inf, partial rows NaN, as
    an unwritten split leaves them) and token 0 with no keys at all, plus W_UV."""
    rng = np.random.default_rng(seed)
    o_part = wl.round_bf16(rng.standard_normal((T, H, S, d_cg)).astype(np.float32))
    lse = (rng.standard_normal((T, H, S)) * 3).astype(np.float32)
    empty = rng.random((T, H, S)) < 1 / 3
    empty[0] = True
    lse[empty] = -np.inf
    o_part[empty] = np.nan
    w_uv = wl.round_bf16((rng.standard_normal((H, d_hc, d_cg)) / np.sqrt(d_cg)).astype(np.float32))
    return o_part, lse, w_uv


def _dev(x, dt=torch.bfloat16):
    return torch.from_numpy(x).to("cuda").to(dt)


# (T, H, d_cg, S, d_hc): every fused instantiation (d_cg 512: S <= 8 and <= 16; d_cg 256:
# S <= 16 and <= 32), one and several 16-row blocks with ragged tails, a head count that
# is not a multiple of 8 (plain workgroup order) and d_hc = 64 and 192.
FUSED = [(16, 128, 512, 8, 128), (37, 128, 512, 16, 128), (5, 128, 512, 1, 128),
         (96, 128, 512, 5, 128), (33, 128, 256, 32, 128), (16, 128, 256, 12, 128),
         (20, 8, 512, 9, 64), (7, 12, 256, 3, 192)]


@pytest.mark.parametrize("T,H,d_cg,S,d_hc", FUSED)
def test_fused_equals_the_two_calls_bitwise(T, H, d_cg, S, d_hc):
    groups = 512 // d_cg
    assert mla.combine_up_v_fused(H, groups, d_hc, d_cg * groups, S)
    o_part, lse, w_uv = _partials(T, H, S, d_cg, d_hc, seed=T * 7 + S)
    op, lp, w = _dev(o_part), torch.from_numpy(lse).to("cuda"), _dev(w_uv)
    # the two calls
    lse_ref = torch.empty((T, H), dtype=torch.float32, device="cuda")
    o_ref = mla.combine(op, lp, lse_out=lse_ref)
    out_ref = mla.up_v(o_ref, w, groups=groups)
    # one call, with the merged rows written, then without them
    o_lat = torch.full((T, H, d_cg), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse_a = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    out_a = mla.combine_up_v(op, lp, w, o_latent=o_lat, lse_out=lse_a, groups=groups)
    lse_b = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    out_b = mla.combine_up_v(op, lp, w, lse_out=lse_b, groups=groups)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_ref) and torch.equal(out_b, out_ref)
    assert torch.equal(o_lat, o_ref)
    assert torch.equal(lse_a, lse_ref) and torch.equal(lse_b, lse_ref)
    assert torch.all(out_a[0] == 0) and torch.all(torch.isneginf(lse_a[0]))


@pytest.mark.parametrize("T,H,d_cg,S,d_hc", [(16, 128, 512, 8, 128), (37, 128, 256, 20, 128)])
def test_fused_against_oracle(T, H, d_cg, S, d_hc):
    """out against the oracle's fp64 merge followed by W_UV (the merged rows rounded to
    bf16 in between, as the library stores o_latent)."""
    groups = 512 // d_cg
    o_part, lse, w_uv = _partials(T, H, S, d_cg, d_hc, seed=1000 + T + S)
    out = mla.combine_up_v(_dev(o_part), torch.from_numpy(lse).to("cuda"), _dev(w_uv), groups=groups)
    torch.cuda.synchronize()
    ref_o, _ = om.merge_splits(o_part, lse)
    ref = om.up_v_reference(wl.round_bf16(ref_o.astype(np.float32)), w_uv)
    got = _f64(out).ravel()
    r = np.asarray(ref, np.float64).ravel()
    err = np.max(np.abs(got - r)) / np.max(np.abs(r))
    cos = float(got @ r / (np.linalg.norm(got) * np.linalg.norm(r)))
    parity_log.record("out (merge + up_v)", err, cos, None, tol=NORM_TOL, cos_tol=COS_TOL)
    assert err <= NORM_TOL and cos >= COS_TOL, (err, cos)


@pytest.mark.parametrize("T,H,d_cg,S,d_hc", [(9, 128, 512, 17, 128), (9, 128, 512, 8, 80)])
def test_uncovered_shapes_run_the_two_calls(T, H, d_cg, S, d_hc):
    """17 splits of 512 columns, or d_hc = 80: the call goes through o_latent (required)
    and gives the two calls' results."""
    assert not mla.combine_up_v_fused(H, 1, d_hc, d_cg, S)
    o_part, lse, w_uv = _partials(T, H, S, d_cg, d_hc, seed=99 + S + d_hc)
    op, lp, w = _dev(o_part), torch.from_numpy(lse).to("cuda"), _dev(w_uv)
    with pytest.raises(mla.MLAError):
        mla.combine_up_v(op, lp, w)
    o_ref = mla.combine(op, lp)
    out_ref = mla.up_v(o_ref, w)
    o_lat = torch.empty((T, H, d_cg), dtype=torch.bfloat16, device="cuda")
    out = mla.combine_up_v(op, lp, w, o_latent=o_lat)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref) and torch.equal(o_lat, o_ref)
