"""Plain CPU float64 oracle for decode-phase Multi-head Latent Attention (MLA).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in ``oracle/``.
The product path (the HIP library and its Python binding) never calls it, and
this module imports nothing from the product package: it receives plain numpy
arrays and returns plain numpy arrays.

Sources (pages are cited by address and section):

* P3 = www.nxmr.cn/news/151634 (MLA operators: matrix absorption, paged latent
  cache).  §1 fixes what one token stores per layer: a 512-d latent c_KV plus a
  64-d decoupled RoPE key k_R, 576 elements in total, i.e. 1.125 KB in bf16
  versus 64 KB for 128 heads x 128 dims of K and V.  §1 also states that the
  latent carries content and the 64-d shared vector carries position, in fully
  separate subspaces.  §3 lists the dimensions (128 heads, d_hc = 128,
  d_c = 512, d_R = 64), page_size 64 and an fp32 RoPE compute dtype.  §4 gives
  the two score paths that must agree -- "naive" (decompress K from the latent,
  then q.K) and "absorbed" (fold W_UK into the query, then q_abs.c_KV) -- both
  with the scale 1/sqrt(d_hc + d_R), and the advice that the RoPE table be
  generated and applied in fp32.
* P2 = m.xxqk.cn/news/443191 (attention from MHA to MoBA), §2.4: K and V are
  jointly compressed into a low-dimensional latent and mapped back up to full
  K and V when needed; the cached latent is 2.25x the size of an MQA cache.
  §2.5 names softmax attention.

What is computed here is the *non-absorbed* definition, written out directly:

    K_h = c @ W_UK[h]^T          (reconstruct per-head content keys, [L, d_hc])
    V_h = c @ W_UV[h]^T          (reconstruct per-head values,       [L, d_hc])
    s_j = (q_c[h] . K_h[j] + RoPE(q_R[h], pos) . k_R[j]) * scale
    p   = softmax(s over visible keys)
    out = sum_j p_j V_h[j]

The absorbed method reaches exactly this result (up to rounding order) because
absorption is only re-association of matrix products, so the definition is the
oracle.  Readings taken where the pages are silent (each also listed in the
design notes):

* softmax: standard softmax with max subtraction over the visible keys (P2 §2.5
  names softmax attention; the MLA pages never write it out).
* scale: 1/sqrt(d_hc + d_R) for every shape (P3 §4).
* W_UK and W_UV are both laid out [H, d_hc, d_c'] ("hdc" in P3 §4's einsum);
  the value head dimension equals d_hc (P3 §1: K/V are 128 heads x 128 dims).
  There is no output projection.
* RoPE: k_R is stored already rotated (it "carries position", P3 §1); the
  cache append (``append_rows`` / ``append_to_pool`` below) rotates a new
  token's key at its own position, the position its query sits at.  The query's q_R is rotated at its
  absolute position with interleaved pairs (2k, 2k+1) and angle pos * theta_k,
  theta_k = base^(-2k/d_R).  ``rope_base=None`` means no rotation, which is the
  P3 §4 check script's setting.
* positions: query i (0-based) of a sequence with L keys (L already includes the
  q_len new tokens) and q_len queries sits at pos = L - q_len + i; with the
  causal flag it sees keys j <= pos, otherwise all L keys.
* grouped latent (GLA, P1 = www.hotelren.com/news/5324130 §1): with G groups,
  head h belongs to group g = h // (H/G) and uses latent columns
  [g*d_c/G, (g+1)*d_c/G); k_R is shared by every head.
"""
from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------------------
# Cache arithmetic (P3 §1, §3, §5; P2 §2.4)
# --------------------------------------------------------------------------


def latent_row_elements(d_c: int, d_R: int) -> int:
    """Elements one token stores per layer in the latent cache: c_KV plus k_R (P3 §1)."""
    return d_c + d_R


def latent_row_bytes(d_c: int, d_R: int, elem_bytes: int = 2) -> int:
    """Bytes per token per layer of the latent cache (P3 §1: bf16 -> 2 bytes/element)."""
    return latent_row_elements(d_c, d_R) * elem_bytes


def mha_row_bytes(heads: int, d_head: int, elem_bytes: int = 2) -> int:
    """Bytes per token per layer of a full MHA cache: K and V for every head (P3 §1)."""
    return 2 * heads * d_head * elem_bytes


def mqa_row_elements(d_head: int) -> int:
    """Elements per token per layer of an MQA cache: one shared K and one V (P2 §2.2-2.4)."""
    return 2 * d_head


def page_bytes(page_size: int, d_c: int, d_R: int, elem_bytes: int = 2) -> int:
    """Bytes in one page of the paged latent cache (P3 §3: page_size 64 -> about 72 KB)."""
    return page_size * latent_row_bytes(d_c, d_R, elem_bytes)


def staged_tile_bytes(tile_tokens: int, d_c: int, d_R: int, stages: int, elem_bytes: int = 2) -> int:
    """On-chip bytes for `stages` buffered tiles of `tile_tokens` latent rows (P3 §5)."""
    return (tile_tokens * d_c + tile_tokens * d_R) * elem_bytes * stages


# --------------------------------------------------------------------------
# RoPE (P3 §1 decoupled position key, §3/§4 fp32 table; reading above)
# --------------------------------------------------------------------------


def rope_angles(positions: np.ndarray, d_R: int, base: float) -> np.ndarray:
    """Angles pos * theta_k for k in [0, d_R/2), theta_k = base^(-2k/d_R); float64 [n, d_R/2]."""
    k = np.arange(d_R // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * k / d_R)
    return np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]


def rope_rotate(x: np.ndarray, pos: int, base: float | None) -> np.ndarray:
    """Rotate the interleaved pairs (x[2k], x[2k+1]) of a d_R vector by pos*theta_k.

    ``base is None`` leaves x unchanged (no positional rotation).
    """
    x = np.asarray(x, dtype=np.float64)
    if base is None:
        return x.copy()
    d_R = x.shape[-1]
    ang = rope_angles(np.array([pos]), d_R, base)[0]
    c, s = np.cos(ang), np.sin(ang)
    even, odd = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = even * c - odd * s
    out[..., 1::2] = even * s + odd * c
    return out


# --------------------------------------------------------------------------
# Score paths of P3 §4 (used for the absorption identity)
# --------------------------------------------------------------------------


def naive_scores(q_c, q_r_rot, c, k_r, w_uk_h, scale):
    """Path A of P3 §4 for one head: decompress K = c W_UK^T, then (q_c.K + q_R.k_R)*scale."""
    k_h = np.asarray(c, np.float64) @ np.asarray(w_uk_h, np.float64).T       # [L, d_hc]
    return (k_h @ np.asarray(q_c, np.float64) + np.asarray(k_r, np.float64) @ q_r_rot) * scale


def absorbed_scores(q_c, q_r_rot, c, k_r, w_uk_h, scale):
    """Path B of P3 §4 for one head: q_abs = q_c W_UK, then (q_abs.c + q_R.k_R)*scale."""
    q_abs = np.asarray(q_c, np.float64) @ np.asarray(w_uk_h, np.float64)    # [d_c']
    return (np.asarray(c, np.float64) @ q_abs + np.asarray(k_r, np.float64) @ q_r_rot) * scale


# --------------------------------------------------------------------------
# The decode step, non-absorbed
# --------------------------------------------------------------------------


def default_scale(d_hc: int, d_R: int) -> float:
    """Softmax scale 1/sqrt(d_hc + d_R) (P3 §4)."""
    return 1.0 / math.sqrt(d_hc + d_R)


def mla_decode(q_c, q_r, latents, w_uk, w_uv, cu_q, *, groups=1, d_c=None,
               rope_base=None, scale=None, causal=True, heads_subset=None,
               seq_subset=None):
    """Non-absorbed MLA decode over logical (un-paged) per-sequence latent rows.

    Arguments (all numpy; anything float is upcast to float64):
      q_c     [T, H, d_hc]   content queries (before absorption)
      q_r     [T, H, d_R]    RoPE queries (before rotation)
      latents list of B arrays [L_b, d_c + d_R]: row j = [c_KV_j | k_R_j]
      w_uk    [H, d_hc, d_c/G]
      w_uv    [H, d_hc, d_c/G]
      cu_q    [B+1] query offsets: sequence b owns query rows cu_q[b]:cu_q[b+1]
    Keyword arguments: groups G, d_c (defaults to G * w_uk.shape[2]), rope_base
    (None = no rotation), scale (None = 1/sqrt(d_hc + d_R)), causal,
    heads_subset / seq_subset (restrict the work; other entries stay NaN).

    Returns a dict with
      out      [T, H, d_hc]  sum_j p_j V_h[j]
      o_latent [T, H, d_c/G] sum_j p_j c_j   (the latent-space attention output)
      lse      [T, H]        log sum_j exp(s_j)
    """
    q_c = np.asarray(q_c, np.float64)
    q_r = np.asarray(q_r, np.float64)
    w_uk = np.asarray(w_uk, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    T, H, d_hc = q_c.shape
    d_R = q_r.shape[2]
    d_cg = w_uk.shape[2]
    if d_c is None:
        d_c = d_cg * groups
    assert d_c == d_cg * groups and H % groups == 0
    heads_per_group = H // groups
    if scale is None:
        scale = default_scale(d_hc, d_R)
    cu_q = np.asarray(cu_q, np.int64)
    B = len(latents)
    assert cu_q.shape[0] == B + 1 and cu_q[-1] == T

    out = np.full((T, H, d_hc), np.nan)
    o_lat = np.full((T, H, d_cg), np.nan)
    lse = np.full((T, H), np.nan)
    heads = range(H) if heads_subset is None else heads_subset
    seqs = range(B) if seq_subset is None else seq_subset
    for b in seqs:
        rows = np.asarray(latents[b], np.float64)
        L = rows.shape[0]
        assert rows.shape[1] == d_c + d_R
        k_r = rows[:, d_c:]
        q_len = int(cu_q[b + 1] - cu_q[b])
        for h in heads:
            g = h // heads_per_group
            c = rows[:, g * d_cg:(g + 1) * d_cg]
            k_h = c @ w_uk[h].T            # [L, d_hc]  reconstructed keys
            v_h = c @ w_uv[h].T            # [L, d_hc]  reconstructed values
            for i in range(q_len):
                t = int(cu_q[b]) + i
                pos = L - q_len + i
                n_vis = min(L, pos + 1) if causal else L
                if n_vis <= 0:
                    out[t, h] = 0.0
                    o_lat[t, h] = 0.0
                    lse[t, h] = -np.inf
                    continue
                qr = rope_rotate(q_r[t, h], pos, rope_base)
                s = (k_h[:n_vis] @ q_c[t, h] + k_r[:n_vis] @ qr) * scale
                m = s.max()
                e = np.exp(s - m)
                z = e.sum()
                p = e / z
                out[t, h] = p @ v_h[:n_vis]
                o_lat[t, h] = p @ c[:n_vis]
                lse[t, h] = m + math.log(z)
    return {"out": out, "o_latent": o_lat, "lse": lse}


def merge_splits(o_parts, lses):
    """Log-sum-exp merge of split-KV partial results.  None of the pages mentions a
    split of the keys or a merge of partial results: the split-KV decode with a separate
    log-sum-exp combine is this library's own reading of the decode task, and the merge
    below is derived from the softmax definition alone (softmax over the union of
    disjoint key sets, written through each set's normaliser).  o_parts [..., S, d] holds each split's softmax-
    normalised output over its own keys and lses [..., S] the natural-log log-sum-exp of
    its scaled scores; a split with lse = -inf holds no keys and its partial never
    enters (it may be unwritten).  With M = max_s lse_s and w_s = exp(lse_s - M):
    out = sum_s w_s o_s / sum_s w_s, lse = M + log sum_s w_s.  A row with no keys at
    all gives out = 0 and lse = -inf.  float64."""
    o = np.asarray(o_parts, np.float64)
    lse = np.asarray(lses, np.float64)
    empty = np.isneginf(lse)
    m = np.max(lse, axis=-1)
    has = ~np.isneginf(m)
    w = np.where(empty, 0.0, np.exp(lse - np.where(has, m, 0.0)[..., None]))
    z = w.sum(axis=-1)
    o = np.where(empty[..., None], 0.0, o)
    out = np.einsum("...s,...sd->...d", w, o) / np.where(has, z, 1.0)[..., None]
    return out, np.where(has, m + np.log(np.where(has, z, 1.0)), -np.inf)


def reconstruct_kv(latent, w_uk, w_uv):
    """The decompressed (non-absorbed) branch's first step (P3 §4 path A; P2 §2.4: K and V
    are mapped back up from the latent): per-head keys and values of latent rows
    c [n, d_c'], K[j,h,:] = W_UK[h] c_j and V[j,h,:] = W_UV[h] c_j, float64 [n, H, d_hc]
    each."""
    c = np.asarray(latent, np.float64)
    w_uk = np.asarray(w_uk, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    return np.einsum("hdc,jc->jhd", w_uk, c), np.einsum("hdc,jc->jhd", w_uv, c)


def absorb_reference(q_c, w_uk):
    """q_abs[t,h,:] = q_c[t,h,:] @ W_UK[h]  (P3 §4 path B, first product), float64."""
    q_c = np.asarray(q_c, np.float64)
    w_uk = np.asarray(w_uk, np.float64)
    return np.einsum("thd,hdc->thc", q_c, w_uk)


def up_v_reference(o_latent, w_uv):
    """out[t,h,:] = W_UV[h] @ o_latent[t,h,:]  (P2 §2.4 up-projection), float64."""
    o_latent = np.asarray(o_latent, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    return np.einsum("hdc,thc->thd", w_uv, o_latent)


def softmax_rows(q_c, q_r, latent, w_uk_h, pos, *, rope_base=None, scale=None, causal=True,
                 group_cols=None):
    """Softmax probabilities of one (sequence, head, query) row, float64 [n_visible]."""
    q_c = np.asarray(q_c, np.float64)
    rows = np.asarray(latent, np.float64)
    d_R = np.asarray(q_r).shape[-1]
    d_c = rows.shape[1] - d_R
    cols = slice(0, d_c) if group_cols is None else group_cols
    if scale is None:
        scale = default_scale(q_c.shape[-1], d_R)
    n_vis = min(rows.shape[0], pos + 1) if causal else rows.shape[0]
    qr = rope_rotate(q_r, pos, rope_base)
    s = naive_scores(q_c, qr, rows[:n_vis, cols], rows[:n_vis, d_c:], w_uk_h, scale)
    e = np.exp(s - s.max())
    return e / e.sum()


# --------------------------------------------------------------------------
# Latent-cache append (P3 §1: what one token stores per layer is its latent c_KV and
# its decoupled RoPE key, the key being the part that carries the token's position;
# P3 §3: 64-token pages; P3 §3/§4: RoPE computed in fp32 -- here in float64)
# --------------------------------------------------------------------------


def new_token_positions(seq_lens, cu_q):
    """Absolute position of every new token, int64 [T].

    Sequence b owns packed rows cu_q[b] .. cu_q[b+1]-1; its length seq_lens[b] already
    counts its q_len new tokens, so new token i sits at seq_lens[b] - q_len + i (the same
    position its query is rotated at)."""
    cu_q = np.asarray(cu_q, np.int64)
    seq_lens = np.asarray(seq_lens, np.int64)
    pos = np.empty(int(cu_q[-1]), np.int64)
    for b in range(len(seq_lens)):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        for i in range(q1 - q0):
            pos[q0 + i] = seq_lens[b] - (q1 - q0) + i
    return pos


def append_rows(c_kv_new, k_r_new, seq_lens, cu_q, rope_base):
    """Cache rows of the new tokens, float64 [T, d_c + d_R]: the latent unchanged, then
    the RoPE key rotated at the token's own position (``rope_base=None``: unrotated)."""
    c = np.asarray(c_kv_new, np.float64)
    k = np.asarray(k_r_new, np.float64)
    pos = new_token_positions(seq_lens, cu_q)
    rows = np.empty((c.shape[0], c.shape[1] + k.shape[1]), np.float64)
    for t in range(c.shape[0]):
        rows[t, :c.shape[1]] = c[t]
        rows[t, c.shape[1]:] = rope_rotate(k[t], int(pos[t]), rope_base)
    return rows


def append_to_pool(pool, page_table, seq_lens, cu_q, c_kv_new, k_r_new, rope_base,
                   page_size=64):
    """The paged pool after the append, float64 [P, page_size, d_c + d_R] (a copy).

    Logical row ``pos`` of sequence b lives in physical page page_table[b][pos // page_size],
    slot pos % page_size; every other slot keeps its content."""
    out = np.array(pool, dtype=np.float64, copy=True)
    rows = append_rows(c_kv_new, k_r_new, seq_lens, cu_q, rope_base)
    pos = new_token_positions(seq_lens, cu_q)
    cu_q = np.asarray(cu_q, np.int64)
    for b in range(len(seq_lens)):
        for t in range(int(cu_q[b]), int(cu_q[b + 1])):
            page = int(page_table[b][int(pos[t]) // page_size])
            out[page, int(pos[t]) % page_size] = rows[t]
    return out
