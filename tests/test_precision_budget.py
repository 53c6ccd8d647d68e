"""Where the bf16 path's error against the fp64 oracle comes from (CPU only).

The GPU path rounds to bf16 at six points: the absorbed query q_abs (an output of
mla_absorb_q), the rotated q_R (parked in LDS as an MFMA operand), the softmax weights
P (MFMA operand), each split's partial output, o_latent (output of mla_combine) and the
final output.  This test emulates that pipeline in float64 with each rounding switched
on alone and all together, on a DeepSeek-V3-shaped batch (2 sequences of 4096 keys,
128 heads, 8 splits), and checks that the terms add up to the 1 - cos the GPU reaches
on the same shape (about 5e-6) and stay under the 1e-5 bar.  It is the error budget
behind keeping the split partials in bf16: they contribute about a ninth of the total.
"""
import numpy as np
import pytest

import oracle.mla_oracle as om
from mla_latent_kv_09_amd import workloads as wl

ROUNDINGS = ("q_abs", "q_r", "p", "part", "o_latent", "out")


def _rb(x):
    return wl.round_bf16(np.asarray(x, np.float32)).astype(np.float64)


def _emulate(w, on, splits=8):
    cfg = w.cfg
    H = cfg.heads
    outs = []
    for b in range(cfg.batch):
        rows = np.asarray(w.latents[b], np.float64)
        L = rows.shape[0]
        c, kr = rows[:, :cfg.d_c], rows[:, cfg.d_c:]
        pos = L - 1
        q_abs = np.einsum("hd,hdc->hc", w.q_c[b].astype(np.float64), w.w_uk.astype(np.float64))
        q_abs = _rb(q_abs) if "q_abs" in on else q_abs
        qr = np.stack([om.rope_rotate(w.q_r[b, h], pos, cfg.rope_base) for h in range(H)])
        qr = _rb(qr) if "q_r" in on else qr
        s = (q_abs @ c.T + qr @ kr.T) * om.default_scale(cfg.d_hc, cfg.d_R)
        parts, lses = [], []
        for keys in np.array_split(np.arange(L), splits):
            m = s[:, keys].max(1, keepdims=True)
            p = np.exp(s[:, keys] - m)
            l = p.sum(1, keepdims=True)
            o = (_rb(p) if "p" in on else p) @ c[keys] / l
            parts.append(_rb(o) if "part" in on else o)
            lses.append((m + np.log(l))[:, 0])
        o, _ = om.merge_splits(np.stack(parts, 1), np.stack(lses, 1))
        o = _rb(o) if "o_latent" in on else o
        out = np.einsum("hdc,hc->hd", w.w_uv.astype(np.float64), o)
        outs.append(_rb(out) if "out" in on else out)
    return np.stack(outs)


def _one_minus_cos(a, b):
    a, b = a.ravel(), b.ravel()
    return 1.0 - float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


@pytest.fixture(scope="module")
def budget():
    cfg = wl.CONFIGS["dsv3_b16_l4096"].replace(batch=2)
    w = wl.make_workload(cfg)
    ref = om.mla_decode(w.q_c, w.q_r, w.latents, w.w_uk, w.w_uv, w.cu_q,
                        rope_base=cfg.rope_base)["out"]
    terms = {r: _one_minus_cos(_emulate(w, {r}), ref) for r in ROUNDINGS}
    total = _one_minus_cos(_emulate(w, set(ROUNDINGS)), ref)
    none = _one_minus_cos(_emulate(w, set()), ref)
    return terms, total, none


def test_emulation_without_roundings_is_the_oracle(budget):
    assert budget[2] < 1e-14


def test_rounding_terms_add_up_and_stay_under_the_bar(budget):
    terms, total, _ = budget
    for r, v in terms.items():
        print(f"{r:>9}: 1-cos {v:.2e}")
    print(f"      all: 1-cos {total:.2e}")
    # each rounding contributes on the order of (2^-9)^2 / 3 per element, scaled by how
    # it propagates; the three roundings of ABI tensors (q_abs, o_latent, out) dominate
    assert all(0 < v < 2e-6 for v in terms.values())
    assert max(terms, key=terms.get) in ("q_abs", "o_latent", "out")
    assert terms["part"] < 0.15 * total
    # independent roundings: the total is close to the sum of the terms
    assert abs(total - sum(terms.values())) < 0.15 * total
    assert total < 0.7e-5
