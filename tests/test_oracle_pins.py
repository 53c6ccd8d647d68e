"""Pins for the CPU oracle: facts fixed by the pages or by mathematics, not by the oracle itself.

Each pin is chosen so that a plausible mistake in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a wrong scale) fails at least one of
them; ``test_planted_mistakes_are_caught`` plants such mistakes and checks that.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.mla_oracle as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers

def _rand_problem(seed, *, B=2, H=4, d_hc=6, d_c=10, d_R=4, G=1, lens=(37, 70), q_lens=(1, 2),
                  w_std=0.4):
    rng = np.random.default_rng(seed)
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    T = int(cu_q[-1])
    q_c = rng.standard_normal((T, H, d_hc))
    q_r = rng.standard_normal((T, H, d_R))
    latents = [rng.standard_normal((L, d_c + d_R)) for L in lens[:B]]
    w_uk = rng.standard_normal((H, d_hc, d_c // G)) * w_std
    w_uv = rng.standard_normal((H, d_hc, d_c // G)) * w_std
    return dict(q_c=q_c, q_r=q_r, latents=latents, w_uk=w_uk, w_uv=w_uv, cu_q=cu_q, groups=G)


def _rotate_complex(x, pos, base):
    """RoPE written as complex multiplication: (x0 + i x1) * exp(i pos theta_k)."""
    d = len(x)
    z = np.array([complex(x[2 * k], x[2 * k + 1]) for k in range(d // 2)])
    th = np.array([base ** (-2.0 * k / d) for k in range(d // 2)])
    z = z * np.exp(1j * pos * th)
    out = np.empty(d)
    out[0::2], out[1::2] = z.real, z.imag
    return out


def _brute_force(p, *, rope_base, causal=True):
    """Scalar loops, absorbed association, no BLAS: an independent route to the same numbers."""
    q_c, q_r, latents, w_uk, w_uv, cu_q, G = (p[k] for k in
                                             ("q_c", "q_r", "latents", "w_uk", "w_uv", "cu_q", "groups"))
    T, H, d_hc = q_c.shape
    d_R = q_r.shape[2]
    d_cg = w_uk.shape[2]
    out = np.zeros((T, H, d_hc))
    lse = np.zeros((T, H))
    for b, rows in enumerate(latents):
        L = rows.shape[0]
        ql = int(cu_q[b + 1] - cu_q[b])
        for i in range(ql):
            t = int(cu_q[b]) + i
            pos = L - ql + i
            for h in range(H):
                g = h // (H // G)
                qa = [sum(q_c[t, h, d] * w_uk[h, d, c] for d in range(d_hc)) for c in range(d_cg)]
                qr = _rotate_complex(q_r[t, h], pos, rope_base) if rope_base else q_r[t, h]
                nv = pos + 1 if causal else L
                s = []
                for j in range(nv):
                    acc = sum(qa[c] * rows[j, g * d_cg + c] for c in range(d_cg))
                    acc += sum(qr[r] * rows[j, G * d_cg + r] for r in range(d_R))
                    s.append(acc / math.sqrt(d_hc + d_R))
                z = sum(math.exp(v) for v in s)
                lse[t, h] = math.log(z)
                ol = [sum(math.exp(s[j]) / z * rows[j, g * d_cg + c] for j in range(nv))
                      for c in range(d_cg)]
                for d in range(d_hc):
                    out[t, h, d] = sum(w_uv[h, d, c] * ol[c] for c in range(d_cg))
    return out, lse


def _run(p, **kw):
    return om.mla_decode(p["q_c"], p["q_r"], p["latents"], p["w_uk"], p["w_uv"], p["cu_q"],
                         groups=p["groups"], **kw)


# ---------------------------------------------------------------- page arithmetic

def test_cache_arithmetic_matches_pages():
    pins = {e["id"]: e for e in json.load(open(os.path.join(GOLDEN, "cache_arithmetic.json")))["pins"]}
    kib = 1024.0
    assert 128 * 128 == pins["mha_dims_per_token"]["value"]
    assert om.latent_row_elements(512, 64) == pins["latent_elements_per_token"]["value"]
    assert om.latent_row_bytes(512, 64) / kib == pins["latent_kb_per_token_bf16"]["value"]
    assert om.mha_row_bytes(128, 128) / kib == pins["mha_kb_per_token_bf16"]["value"]
    comp = 100.0 * (1.0 - om.latent_row_bytes(512, 64) / om.mha_row_bytes(128, 128))
    assert round(comp, 2) == pins["compression_percent"]["value"]
    assert om.latent_row_elements(512, 64) / om.mqa_row_elements(128) == pins["latent_over_mqa"]["value"]
    assert om.page_bytes(64, 512, 64) / kib == pins["page_kb_page_size_64"]["value"]
    assert om.page_bytes(16, 512, 64) / kib == pins["page_kb_page_size_16"]["value"]
    assert om.staged_tile_bytes(64, 512, 64, 3) / kib == pins["tile64_x3_stages_kb"]["value"]
    assert om.staged_tile_bytes(64, 512, 64, 3) <= pins["hopper_smem_kb"]["value"] * kib
    # doubling the tile overflows the per-SM limit, as the page reports
    assert om.staged_tile_bytes(128, 512, 64, 3) > pins["hopper_smem_kb"]["value"] * kib


def test_default_scale_is_one_over_sqrt_192():
    assert om.default_scale(128, 64) == 1.0 / math.sqrt(192.0)
    assert abs(om.default_scale(32, 16) - 1.0 / math.sqrt(48.0)) < 1e-17


# ---------------------------------------------------------------- absorption identity (P3 §4)

@pytest.mark.parametrize("d_hc,d_c,d_R", [(128, 512, 64), (7, 13, 4)])
def test_absorption_identity_fp64(d_hc, d_c, d_R):
    rng = np.random.default_rng(42)
    S = 257
    q_c = rng.standard_normal(d_hc)
    q_r = rng.standard_normal(d_R)
    w = rng.standard_normal((d_hc, d_c))
    c = rng.standard_normal((S, d_c))
    k_r = rng.standard_normal((S, d_R))
    sc = om.default_scale(d_hc, d_R)
    a = om.naive_scores(q_c, q_r, c, k_r, w, sc)
    b = om.absorbed_scores(q_c, q_r, c, k_r, w, sc)
    assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(a))
    # the same scores from a third route: explicit scalar sums on a few keys
    for j in (0, 100, S - 1):
        ref = sum(q_c[d] * sum(c[j, e] * w[d, e] for e in range(d_c)) for d in range(d_hc))
        ref = (ref + float(q_r @ k_r[j])) * sc
        assert abs(ref - a[j]) <= 1e-11 * max(1.0, abs(ref))


# ---------------------------------------------------------------- RoPE

def test_rope_closed_forms():
    # d_R = 2, base anything: theta_0 = 1, so the pair turns by `pos` radians
    x = np.array([1.0, 0.0])
    y = om.rope_rotate(x, 3, 10000.0)
    assert np.allclose(y, [math.cos(3.0), math.sin(3.0)], atol=1e-15)
    # pos 0 is the identity; base None is the identity
    v = np.random.default_rng(1).standard_normal(64)
    assert np.array_equal(om.rope_rotate(v, 0, 10000.0), v)
    assert np.array_equal(om.rope_rotate(v, 77, None), v)
    # second pair of a d_R = 4 vector turns by pos * base^(-1/2)
    x4 = np.array([0.0, 0.0, 1.0, 0.0])
    y4 = om.rope_rotate(x4, 5, 100.0)
    assert np.allclose(y4, [0, 0, math.cos(0.5), math.sin(0.5)], atol=1e-15)


def test_rope_matches_complex_rotation_and_is_relative():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for pos in (1, 17, 4095, 65535):
        assert np.allclose(om.rope_rotate(q, pos, 10000.0), _rotate_complex(q, pos, 10000.0),
                           atol=1e-9)
        assert abs(np.linalg.norm(om.rope_rotate(q, pos, 10000.0)) - np.linalg.norm(q)) < 1e-12
    # <R(m) q, R(n) k> depends only on m - n
    d1 = om.rope_rotate(q, 50, 10000.0) @ om.rope_rotate(k, 30, 10000.0)
    d2 = om.rope_rotate(q, 1020, 10000.0) @ om.rope_rotate(k, 1000, 10000.0)
    assert abs(d1 - d2) < 1e-9


# ---------------------------------------------------------------- whole decode step

@pytest.mark.parametrize("rope", [None, 10000.0])
@pytest.mark.parametrize("G", [1, 2])
def test_oracle_matches_brute_force(rope, G):
    p = _rand_problem(3 + G, G=G)
    r = _run(p, rope_base=rope)
    bf_out, bf_lse = _brute_force(p, rope_base=rope)
    assert np.max(np.abs(r["out"] - bf_out)) <= 1e-12 * np.max(np.abs(bf_out))
    assert np.max(np.abs(r["lse"] - bf_lse)) <= 1e-12 * np.max(np.abs(bf_lse))


def test_oracle_matches_sdpa_textbook_special_case():
    """Non-absorbed MLA is standard attention with 192-d keys [c W_UK^T, k_R] and values c W_UV^T."""
    p = _rand_problem(7, B=2, H=3, d_hc=16, d_c=24, d_R=8, lens=(65, 130), q_lens=(2, 1))
    base = 10000.0
    r = _run(p, rope_base=base)
    for b, rows in enumerate(p["latents"]):
        L = rows.shape[0]
        ql = int(p["cu_q"][b + 1] - p["cu_q"][b])
        for h in range(3):
            kk = np.concatenate([rows[:, :24] @ p["w_uk"][h].T, rows[:, 24:]], axis=1)
            vv = rows[:, :24] @ p["w_uv"][h].T
            qs, mask = [], []
            for i in range(ql):
                t = int(p["cu_q"][b]) + i
                pos = L - ql + i
                qs.append(np.concatenate([p["q_c"][t, h], _rotate_complex(p["q_r"][t, h], pos, base)]))
                mask.append(np.arange(L) <= pos)
            o = torch.nn.functional.scaled_dot_product_attention(
                torch.tensor(np.array(qs))[None], torch.tensor(kk)[None], torch.tensor(vv)[None],
                attn_mask=torch.tensor(np.array(mask))[None]).numpy()[0]
            got = r["out"][int(p["cu_q"][b]):int(p["cu_q"][b + 1]), h]
            assert np.max(np.abs(got - o)) <= 1e-12 * np.max(np.abs(o))


def test_softmax_rows_sum_to_one_and_lse():
    p = _rand_problem(11)
    rows = p["latents"][1]
    pr = om.softmax_rows(p["q_c"][1, 2], p["q_r"][1, 2], rows, p["w_uk"][2], pos=68, rope_base=10000.0)
    assert pr.shape == (69,)
    assert abs(pr.sum() - 1.0) <= 1e-12 and (pr > 0).all()
    r = _run(p, rope_base=10000.0)
    # o_latent is the same softmax applied to the latent rows
    c = rows[:69, :10]
    assert np.allclose(r["o_latent"][1, 2], pr @ c, rtol=1e-12, atol=1e-13)
    # LSE: exp(s_j - lse) are the probabilities
    s = om.naive_scores(p["q_c"][1, 2], om.rope_rotate(p["q_r"][1, 2], 68, 10000.0), c, rows[:69, 10:],
                        p["w_uk"][2], om.default_scale(6, 4))
    assert np.allclose(np.exp(s - r["lse"][1, 2]), pr, rtol=1e-12, atol=1e-15)


def test_value_path_associativity():
    """W_UV (sum_j p_j c_j) == sum_j p_j (W_UV c_j): the absorbed value path reaches the same output."""
    p = _rand_problem(13, G=2)
    r = _run(p, rope_base=10000.0)
    T, H = r["out"].shape[:2]
    for t in range(T):
        for h in range(H):
            assert np.allclose(p["w_uv"][h] @ r["o_latent"][t, h], r["out"][t, h], rtol=1e-11, atol=1e-12)


def test_closed_form_single_key():
    p = _rand_problem(17, B=1, lens=(1,), q_lens=(1,))
    r = _run(p, rope_base=10000.0)
    c0 = p["latents"][0][0, :10]
    for h in range(4):
        assert np.allclose(r["out"][0, h], p["w_uv"][h] @ c0, rtol=1e-13, atol=1e-14)
        assert np.allclose(r["o_latent"][0, h], c0, rtol=0, atol=1e-15)


def test_closed_form_zero_query_is_uniform_average():
    p = _rand_problem(19, B=1, lens=(50,), q_lens=(1,))
    p["q_c"][:] = 0.0
    p["q_r"][:] = 0.0
    r = _run(p, rope_base=10000.0)
    c = p["latents"][0][:, :10]
    for h in range(4):
        assert np.allclose(r["out"][0, h], p["w_uv"][h] @ c.mean(axis=0), rtol=1e-12, atol=1e-14)
        assert abs(r["lse"][0, h] - math.log(50)) < 1e-13


def test_closed_form_identical_rows():
    p = _rand_problem(23, B=1, lens=(40,), q_lens=(2,))
    p["latents"][0][:] = p["latents"][0][5]
    r = _run(p, rope_base=None)
    for h in range(4):
        assert np.allclose(r["out"][:, h], p["w_uv"][h] @ p["latents"][0][5, :10], rtol=1e-12, atol=1e-14)


def test_causal_row_zero_equals_shorter_decode():
    """Query 0 of a q_len-2 sequence with L keys is a q_len-1 decode over the first L-1 keys."""
    p = _rand_problem(29, B=1, lens=(70,), q_lens=(2,))
    r2 = _run(p, rope_base=10000.0)
    p1 = dict(p, latents=[p["latents"][0][:69]], q_c=p["q_c"][:1], q_r=p["q_r"][:1],
              cu_q=np.array([0, 1]))
    r1 = _run(p1, rope_base=10000.0)
    assert np.allclose(r2["out"][0], r1["out"][0], rtol=1e-13, atol=1e-14)
    # and the non-causal variant lets query 0 see all 70 keys: a different answer
    rn = _run(p, rope_base=10000.0, causal=False)
    assert not np.allclose(rn["out"][0], r1["out"][0])


def test_grouped_latent_is_two_independent_problems():
    p = _rand_problem(31, H=4, d_c=10, G=2)
    r = _run(p, rope_base=10000.0)
    d_cg = 5
    for g in range(2):
        hs = slice(2 * g, 2 * g + 2)
        lat = [np.concatenate([x[:, g * d_cg:(g + 1) * d_cg], x[:, 10:]], axis=1) for x in p["latents"]]
        pg = dict(p, q_c=p["q_c"][:, hs], q_r=p["q_r"][:, hs], latents=lat, w_uk=p["w_uk"][hs],
                  w_uv=p["w_uv"][hs], groups=1)
        rg = _run(pg, rope_base=10000.0)
        assert np.allclose(r["out"][:, hs], rg["out"], rtol=1e-13, atol=1e-14)


def test_subsets_compute_only_what_is_asked():
    p = _rand_problem(37)
    full = _run(p, rope_base=10000.0)
    part = _run(p, rope_base=10000.0, heads_subset=[1, 3], seq_subset=[1])
    t1 = slice(int(p["cu_q"][1]), int(p["cu_q"][2]))
    assert np.array_equal(part["out"][t1, [1, 3]], full["out"][t1, [1, 3]])
    assert np.isnan(part["out"][0]).all()


# ---------------------------------------------------------------- pins have teeth

def _mutant_decode(kind):
    real = om.mla_decode

    def patched(q_c, q_r, latents, w_uk, w_uv, cu_q, **kw):
        q_c = np.asarray(q_c, np.float64)
        if kind == "scale_dhc_only":
            kw["scale"] = 1.0 / math.sqrt(q_c.shape[2])
            return real(q_c, q_r, latents, w_uk, w_uv, cu_q, **kw)
        if kind == "dropped_rope_term":
            return real(q_c, np.zeros_like(np.asarray(q_r, np.float64)), latents, w_uk, w_uv, cu_q, **kw)
        if kind == "w_uk_untransposed":
            # reads W_UK with d_hc and d_c' swapped (only shape-valid when square)
            w = np.asarray(w_uk, np.float64)
            w = w.reshape(w.shape[0], w.shape[2], w.shape[1]).transpose(0, 2, 1)
            return real(q_c, q_r, latents, w, w_uv, cu_q, **kw)
        if kind == "v_from_w_uk":
            return real(q_c, q_r, latents, w_uk, w_uk, cu_q, **kw)
        if kind == "rope_sign":
            orig = om.rope_rotate
            om.rope_rotate = lambda x, pos, base: orig(x, -pos, base)
            try:
                return real(q_c, q_r, latents, w_uk, w_uv, cu_q, **kw)
            finally:
                om.rope_rotate = orig
        raise ValueError(kind)
    return patched


@pytest.mark.parametrize("kind", ["scale_dhc_only", "dropped_rope_term", "w_uk_untransposed",
                                  "v_from_w_uk", "rope_sign"])
def test_planted_mistakes_are_caught(kind):
    p = _rand_problem(41, d_hc=6, d_c=6, d_R=4, lens=(20, 33))
    bad = _mutant_decode(kind)(p["q_c"], p["q_r"], p["latents"], p["w_uk"], p["w_uv"], p["cu_q"],
                               groups=1, rope_base=10000.0)
    bf_out, _ = _brute_force(p, rope_base=10000.0)
    assert np.max(np.abs(bad["out"] - bf_out)) > 1e-6 * np.max(np.abs(bf_out))


def test_projection_references_match_scalar_sums():
    rng = np.random.default_rng(43)
    q = rng.standard_normal((3, 2, 5))
    w = rng.standard_normal((2, 5, 7))
    qa = om.absorb_reference(q, w)
    o = rng.standard_normal((3, 2, 7))
    ov = om.up_v_reference(o, w)
    for t in range(3):
        for h in range(2):
            for c in range(7):
                assert abs(qa[t, h, c] - sum(q[t, h, d] * w[h, d, c] for d in range(5))) < 1e-12
            for d in range(5):
                assert abs(ov[t, h, d] - sum(w[h, d, c] * o[t, h, c] for c in range(7))) < 1e-12
    # the absorbed query against the latent reproduces the naive content score (P3 section 4)
    c = rng.standard_normal((4, 7))
    naive = om.naive_scores(q[1, 1], np.zeros(2), c, np.zeros((4, 2)), w[1], 1.0)
    assert np.allclose(c @ qa[1, 1], naive, rtol=1e-12, atol=1e-12)


def test_merge_of_key_chunks_equals_attention_over_all_keys():
    """The split merge is pinned to the oracle's own softmax over all keys: attention over
    each chunk of the keys separately (no causal mask, no RoPE, so a chunk's scores are
    the same as in the whole), merged by lse, equals attention over all keys.  One chunk
    is empty (lse = -inf, partial NaN: it must not enter)."""
    rng = np.random.default_rng(5)
    H, d_hc, d_c, d_R, L = 4, 8, 16, 4, 23
    q_c = rng.standard_normal((1, H, d_hc))
    q_r = rng.standard_normal((1, H, d_R))
    rows = rng.standard_normal((L, d_c + d_R))
    w_uk = rng.standard_normal((H, d_hc, d_c)) / 4
    w_uv = rng.standard_normal((H, d_hc, d_c)) / 4
    cu = np.array([0, 1])
    full = om.mla_decode(q_c, q_r, [rows], w_uk, w_uv, cu, causal=False)
    bounds = [0, 5, 5, 12, 23]                      # chunk [5, 5) is empty
    parts, lses = [], []
    for a, b in zip(bounds, bounds[1:]):
        if a == b:
            parts.append(np.full((1, H, d_c), np.nan))
            lses.append(np.full((1, H), -np.inf))
            continue
        r = om.mla_decode(q_c, q_r, [rows[a:b]], w_uk, w_uv, cu, causal=False)
        parts.append(r["o_latent"])
        lses.append(r["lse"])
    o, lse = om.merge_splits(np.stack(parts, axis=2), np.stack(lses, axis=2))
    assert np.allclose(o, full["o_latent"], rtol=0, atol=1e-12)
    assert np.allclose(lse, full["lse"], rtol=0, atol=1e-12)
    # no keys anywhere: zero output, -inf lse
    o0, l0 = om.merge_splits(np.full((2, 3, 5), np.nan), np.full((2, 3), -np.inf))
    assert np.all(o0 == 0) and np.all(np.isneginf(l0))


def test_reconstruct_kv_matches_scalar_sums():
    rng = np.random.default_rng(41)
    c = rng.standard_normal((5, 7))
    w_uk = rng.standard_normal((3, 4, 7))
    w_uv = rng.standard_normal((3, 4, 7))
    k, v = om.reconstruct_kv(c, w_uk, w_uv)
    assert k.shape == v.shape == (5, 3, 4)
    for j in range(5):
        for h in range(3):
            for d in range(4):
                assert k[j, h, d] == pytest.approx(sum(w_uk[h, d, x] * c[j, x] for x in range(7)), rel=1e-13)
                assert v[j, h, d] == pytest.approx(sum(w_uv[h, d, x] * c[j, x] for x in range(7)), rel=1e-13)


def test_prefill_shaped_batch_is_causal_attention():
    """A prompt whose every token is a query (q_len = L, the decompressed branch's shape):
    the oracle equals SDPA with the causal triangle over [c W_UK^T | k_R] keys and
    c W_UV^T values, and query i sees exactly keys 0 .. i."""
    p = _rand_problem(43, B=1, H=2, d_hc=8, d_c=12, d_R=4, lens=(70,), q_lens=(70,))
    base = 10000.0
    r = _run(p, rope_base=base)
    rows = p["latents"][0]
    k, v = om.reconstruct_kv(rows[:, :12], p["w_uk"], p["w_uv"])
    for h in range(2):
        kk = np.concatenate([k[:, h], rows[:, 12:]], axis=1)
        qs = np.stack([np.concatenate([p["q_c"][i, h], _rotate_complex(p["q_r"][i, h], i, base)])
                       for i in range(70)])
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(qs)[None], torch.tensor(kk)[None], torch.tensor(v[:, h])[None],
            is_causal=True).numpy()[0]
        assert np.max(np.abs(r["out"][:, h] - o)) <= 1e-12 * np.max(np.abs(o))
    # the first query sees only key 0: its output is that key's value exactly
    assert np.allclose(r["out"][0], v[0], rtol=1e-13, atol=0)
