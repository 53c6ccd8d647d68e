"""Seeded synthetic inputs for paged MLA decode.

This module only draws random numbers, rounds them to the storage dtype and
places latent rows into a paged pool.  It holds none of the attention
arithmetic, so both the HIP path and the CPU oracle can consume what it makes
without sharing any code of the method.

Input recipe (the same for every consumer):

* Every tensor has its own numpy ``PCG64`` stream, seeded by
  ``SeedSequence([seed, tensor_index])`` (the latent rows of sequence b by
  ``SeedSequence([seed, tensor_index, b])``), so adding a tensor or a sequence
  never shifts the draws of another one, and sequences can be drawn in parallel.
* Activations q_c, q_R, c_KV and k_R are standard normal.  Weights W_UK and W_UV
  are normal with standard deviation ``w_std`` (1/sqrt(d_c) unless stated).
* Draws are float32 and then rounded to the storage dtype: bf16 with
  round-to-nearest-even, or kept as float32 for the fp32 workload.  The arrays
  handed out are float32 arrays holding exactly the stored values, plus the
  raw storage (uint16 bf16 bit patterns or float32) for the device.
* Paged pool: sequence b owns ceil(L_b / page_size) pages; the pool holds
  exactly the sum of those, in a uniformly random permutation (identity when
  ``identity_pages``).  Slots past L_b in a sequence's last page are filled with
  NaN so that a kernel which fails to mask them cannot pass.  Unused
  page-table entries are -1.
* Ragged batches draw L_b uniformly from an inclusive integer range and give
  query length 1 to a random half of the sequences and 2 to the rest.
* Cache append inputs (``make_new_tokens``): one latent c_KV [d_c] and one unrotated
  RoPE key k_R [d_R] per new token (T of them, one per query row), standard normal,
  rounded like the rest.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import math
import os
from collections.abc import Sequence
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BF16_NAN_BITS = 0x7FC0

_STREAMS = {
    "q_c": 1, "q_r": 2, "latent": 3, "w_uk": 4, "w_uv": 5,
    "pages": 6, "lengths": 7, "q_lens": 8, "c_kv_new": 9, "k_r_new": 10,
}


def _rng(seed: int, name: str, *sub: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([int(seed), _STREAMS[name], *map(int, sub)])))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if nan.any():
        out[nan] = BF16_NAN_BITS
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the float32 values they encode (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bf16 (RNE), returned as float32."""
    return bf16_bits_to_f32(bf16_bits(x))


@dataclass(frozen=True)
class MLAConfig:
    """Shape and input statistics of one decode workload."""

    name: str
    batch: int
    heads: int
    d_hc: int
    d_c: int
    d_R: int
    groups: int = 1
    dtype: str = "bf16"                 # storage and MFMA operand dtype: "bf16" or "fp32"
    seq_len: Optional[int] = None       # every sequence has this many keys (incl. new tokens)
    seq_len_range: Optional[tuple] = None   # inclusive uniform range for ragged batches
    q_len: int = 1                      # queries per sequence (ignored when q_len_mix)
    q_len_mix: bool = False             # half the sequences q_len 1, the rest 2
    page_size: int = 64
    identity_pages: bool = False
    w_std: Optional[float] = None       # None -> 1/sqrt(d_c)
    causal: bool = True
    rope_base: Optional[float] = 10000.0
    seed: int = 0
    note: str = ""

    @property
    def d_cg(self) -> int:
        return self.d_c // self.groups

    @property
    def row(self) -> int:
        return self.d_c + self.d_R

    @property
    def weight_std(self) -> float:
        return self.w_std if self.w_std is not None else 1.0 / math.sqrt(self.d_c)

    def replace(self, **kw) -> "MLAConfig":
        return dataclasses.replace(self, **kw)


# The five workloads of the decode study.  Names describe the shape.
CONFIGS = {
    "tiny_fp32": MLAConfig(
        name="tiny_fp32", batch=1, heads=16, d_hc=32, d_c=64, d_R=16, dtype="fp32",
        seq_len=256, identity_pages=True, w_std=1.0 / 8.0,
        note="batch 1, q_len 1, 16 heads, d_hc 32, d_c 64, d_R 16, 256 contiguous tokens, fp32"),
    "dsv3_b16_l4096": MLAConfig(
        name="dsv3_b16_l4096", batch=16, heads=128, d_hc=128, d_c=512, d_R=64,
        seq_len=4096,
        note="DeepSeek-V3-shaped layer: batch 16, q_len 1, 128 heads, 4096 tokens, bf16"),
    "long_b16_l65536": MLAConfig(
        name="long_b16_l65536", batch=16, heads=128, d_hc=128, d_c=512, d_R=64,
        seq_len=65536,
        note="long context: batch 16, q_len 1, 128 heads, 65536 tokens (~1.2 GB cache), bf16"),
    "ragged_b64": MLAConfig(
        name="ragged_b64", batch=64, heads=128, d_hc=128, d_c=512, d_R=64,
        seq_len_range=(1024, 32768), q_len_mix=True,
        note="ragged batch 64, lengths U[1024, 32768], q_len 1 or 2 (half each), causal, bf16"),
    "gla2_b32_l16384": MLAConfig(
        name="gla2_b32_l16384", batch=32, heads=128, d_hc=128, d_c=512, d_R=64, groups=2,
        seq_len=16384, w_std=1.0 / 16.0,
        note="grouped latent (2 groups of 64 heads, 256-d slice each + shared 64-d k_R), "
             "batch 32, 16384 tokens, bf16"),
    # The prefill/decode dispatch measurement of the MLA-operators page (§6): batch 8,
    # 4096-token prompts, every prompt token a query (causal), at the 256-row threshold.
    "prefill_b8_l4096": MLAConfig(
        name="prefill_b8_l4096", batch=8, heads=128, d_hc=128, d_c=512, d_R=64,
        seq_len=4096, q_len=4096,
        note="prefill: batch 8, 4096-token prompts, q_len = 4096 (causal), 128 heads, bf16"),
}

CONFIG_ORDER = ["tiny_fp32", "dsv3_b16_l4096", "long_b16_l65536", "ragged_b64", "gla2_b32_l16384"]


class PagedRows(Sequence):
    """Per-sequence logical latent rows [L_b, d_c + d_R] (float32), read back out of
    the paged pool on access, so no second copy of a multi-GB cache is kept."""

    def __init__(self, w: "Workload"):
        self._w = w

    def __len__(self) -> int:
        return len(self._w.seq_lens)

    def __getitem__(self, b):
        if isinstance(b, slice):
            return [self[i] for i in range(*b.indices(len(self)))]
        if b < 0:
            b += len(self)
        if not 0 <= b < len(self):
            raise IndexError(b)
        return gather_sequence(self._w, b)


@dataclass
class Workload:
    """One generated decode step: host arrays shared by the device path and the oracle."""

    cfg: MLAConfig
    seq_lens: np.ndarray        # int32 [B]   keys per sequence (incl. the new tokens)
    q_lens: np.ndarray          # int32 [B]
    cu_q: np.ndarray            # int32 [B+1]
    q_c: np.ndarray             # float32 [T, H, d_hc]   (values exact in the storage dtype)
    q_r: np.ndarray             # float32 [T, H, d_R]
    latents: Sequence           # B x float32 [L_b, d_c + d_R] (PagedRows, or a list)
    w_uk: np.ndarray            # float32 [H, d_hc, d_c/G]
    w_uv: np.ndarray            # float32 [H, d_hc, d_c/G]
    page_table: np.ndarray      # int32 [B, max_pages]   (-1 = unused)
    pool: np.ndarray            # [P, page_size, d_c + d_R]: uint16 bf16 bits or float32
    extras: dict = field(default_factory=dict)

    @property
    def total_q(self) -> int:
        return int(self.cu_q[-1])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def num_pool_pages(self) -> int:
        return int(self.pool.shape[0])

    def storage(self, x: np.ndarray) -> np.ndarray:
        """A float32 array of exact values in its device storage form."""
        return bf16_bits(x) if self.cfg.dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def make_workload(cfg: MLAConfig, *, seed: Optional[int] = None, nan_fill: bool = True) -> Workload:
    """Draw one decode step for ``cfg`` (seed defaults to ``cfg.seed``)."""
    seed = cfg.seed if seed is None else seed
    B, H = cfg.batch, cfg.heads
    rnd = round_bf16 if cfg.dtype == "bf16" else (lambda a: a.astype(np.float32))

    if cfg.seq_len_range is not None:
        lo, hi = cfg.seq_len_range
        seq_lens = _rng(seed, "lengths").integers(lo, hi + 1, size=B).astype(np.int32)
    else:
        seq_lens = np.full(B, cfg.seq_len, dtype=np.int32)
    if cfg.q_len_mix:
        q_lens = np.ones(B, dtype=np.int32)
        q_lens[_rng(seed, "q_lens").permutation(B)[: B // 2]] = 2
    else:
        q_lens = np.full(B, cfg.q_len, dtype=np.int32)
    cu_q = np.zeros(B + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(q_lens)
    T = int(cu_q[-1])

    q_c = rnd(_normal(_rng(seed, "q_c"), (T, H, cfg.d_hc)))
    q_r = rnd(_normal(_rng(seed, "q_r"), (T, H, cfg.d_R)))
    w_uk = rnd(_normal(_rng(seed, "w_uk"), (H, cfg.d_hc, cfg.d_cg), cfg.weight_std))
    w_uv = rnd(_normal(_rng(seed, "w_uv"), (H, cfg.d_hc, cfg.d_cg), cfg.weight_std))

    ps = cfg.page_size
    pages_per_seq = [(int(L) + ps - 1) // ps for L in seq_lens]
    P = int(sum(pages_per_seq))
    perm = np.arange(P) if cfg.identity_pages else _rng(seed, "pages").permutation(P)
    max_pages = max(pages_per_seq) if pages_per_seq else 0
    page_table = np.full((B, max(max_pages, 1)), -1, dtype=np.int32)
    offsets = np.concatenate([[0], np.cumsum(pages_per_seq)]).astype(np.int64)
    for b in range(B):
        page_table[b, :pages_per_seq[b]] = perm[offsets[b]:offsets[b + 1]]

    if cfg.dtype == "bf16":
        pool = np.full((P, ps, cfg.row), BF16_NAN_BITS if nan_fill else 0, dtype=np.uint16)
    else:
        pool = np.full((P, ps, cfg.row), np.nan if nan_fill else 0.0, dtype=np.float32)

    def fill(b: int) -> None:
        L = int(seq_lens[b])
        x = _normal(_rng(seed, "latent", b), (L, cfg.row))
        rows = bf16_bits(x) if cfg.dtype == "bf16" else x
        for k in range(pages_per_seq[b]):
            chunk = rows[k * ps:(k + 1) * ps]
            pool[page_table[b, k], :chunk.shape[0]] = chunk

    workers = min(16, os.cpu_count() or 1, max(1, B))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(fill, range(B)))
    w = Workload(cfg=cfg, seq_lens=seq_lens, q_lens=q_lens, cu_q=cu_q, q_c=q_c, q_r=q_r,
                 latents=[], w_uk=w_uk, w_uv=w_uv, page_table=page_table, pool=pool)
    w.latents = PagedRows(w)
    return w

@dataclass
class NewTokens:
    """The latent rows a decode step appends: one per new token (packed query row)."""

    c_kv: np.ndarray            # float32 [T, d_c]   (values exact in the storage dtype)
    k_r: np.ndarray             # float32 [T, d_R]   before rotation


def make_new_tokens(w: Workload, *, seed: Optional[int] = None,
                    rows: Optional[int] = None) -> NewTokens:
    """Draw the new tokens' c_KV and (unrotated) k_R for workload ``w``: one per query
    row, or ``rows`` of them."""
    cfg = w.cfg
    seed = cfg.seed if seed is None else seed
    rnd = round_bf16 if cfg.dtype == "bf16" else (lambda a: a.astype(np.float32))
    T = w.total_q if rows is None else int(rows)
    return NewTokens(c_kv=rnd(_normal(_rng(seed, "c_kv_new"), (T, cfg.d_c))),
                     k_r=rnd(_normal(_rng(seed, "k_r_new"), (T, cfg.d_R))))


def gather_sequence(w: Workload, b: int) -> np.ndarray:
    """Read sequence b's rows back out of the paged pool (float32), for layout checks."""
    ps = w.cfg.page_size
    L = int(w.seq_lens[b])
    n = (L + ps - 1) // ps
    pages = w.pool[w.page_table[b, :n]].reshape(n * ps, w.cfg.row)[:L]
    return bf16_bits_to_f32(pages) if w.cfg.dtype == "bf16" else pages.astype(np.float32)


def mxfp4_pool(w: Workload, packed: Sequence, scales: Sequence, *, nan_fill: bool = True) -> np.ndarray:
    """Place per-sequence MXFP4 latent codes (uint8 [L_b, d_c / 2], two per byte) and scale
    bytes (uint8 [L_b, d_c / 32]) into MXFP4 cache pages laid out as {codes [64][d_c / 2] |
    k_R [64][d_R] bf16 | scales [64][d_c / 32]}, the k_R rows taken from ``w``'s bf16
    pool.  Pure data placement: the codes and scales are given.  Slots past a sequence's
    end hold 0xFF codes (-6), NaN k_R and the out-of-format scale byte 255 when
    ``nan_fill``.  Returns uint8 [P, 64 (d_c / 2 + 2 d_R + d_c / 32)]."""
    cfg = w.cfg
    if cfg.dtype != "bf16":
        raise ValueError("MXFP4 pages take a bf16 workload's k_R rows")
    ps, d_c, d_R = cfg.page_size, cfg.d_c, cfg.d_R
    cb, sb = d_c // 2, d_c // 32
    P = w.num_pool_pages
    pool = np.zeros((P, ps * (cb + 2 * d_R + sb)), np.uint8)
    code_part = pool[:, : ps * cb].reshape(P, ps, cb)
    rope_part = pool[:, ps * cb: ps * (cb + 2 * d_R)].view(np.uint16).reshape(P, ps, d_R)
    scale_part = pool[:, ps * (cb + 2 * d_R):].reshape(P, ps, sb)
    if nan_fill:
        code_part[...] = 0xFF
        rope_part[...] = BF16_NAN_BITS
        scale_part[...] = 0xFF
    for b in range(len(w.seq_lens)):
        L = int(w.seq_lens[b])
        for k in range((L + ps - 1) // ps):
            pg = int(w.page_table[b, k])
            n = min(ps, L - k * ps)
            code_part[pg, :n] = packed[b][k * ps: k * ps + n]
            scale_part[pg, :n] = scales[b][k * ps: k * ps + n]
            rope_part[pg, :n] = w.pool[pg, :n, d_c:]
    return pool


def fp8_pool(w: Workload, codes: Sequence, scales: Sequence, *, nan_fill: bool = True) -> np.ndarray:
    """Place per-sequence FP8 latent codes (uint8 [L_b, d_c]) and token scales (float32
    [L_b]) into FP8 cache pages laid out as {codes [64][d_c] | k_R [64][d_R] bf16 |
    scales [64] float32}, the k_R rows taken from ``w``'s bf16 pool.  Pure data placement:
    the codes and scales are given.  Slots past a sequence's end hold NaN codes (0x7F),
    NaN k_R and NaN scales when ``nan_fill``.  Returns uint8 [P, 64 (d_c + 2 d_R + 4)]."""
    cfg = w.cfg
    if cfg.dtype != "bf16":
        raise ValueError("FP8 pages take a bf16 workload's k_R rows")
    ps, d_c, d_R = cfg.page_size, cfg.d_c, cfg.d_R
    P = w.num_pool_pages
    pool = np.zeros((P, ps * (d_c + 2 * d_R + 4)), np.uint8)
    code_part = pool[:, : ps * d_c].reshape(P, ps, d_c)
    rope_part = pool[:, ps * d_c: ps * (d_c + 2 * d_R)].view(np.uint16).reshape(P, ps, d_R)
    scale_part = pool[:, ps * (d_c + 2 * d_R):].view(np.float32).reshape(P, ps)
    if nan_fill:
        code_part[...] = 0x7F
        rope_part[...] = BF16_NAN_BITS
        scale_part[...] = np.nan
    for b in range(len(w.seq_lens)):
        L = int(w.seq_lens[b])
        for k in range((L + ps - 1) // ps):
            pg = int(w.page_table[b, k])
            n = min(ps, L - k * ps)
            code_part[pg, :n] = codes[b][k * ps: k * ps + n]
            scale_part[pg, :n] = scales[b][k * ps: k * ps + n]
            rope_part[pg, :n] = w.pool[pg, :n, d_c:]
    return pool
