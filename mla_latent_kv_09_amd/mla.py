"""Thin Python binding of ``libmla_kv.so`` (C ABI in ``include/mla_kv.h``).

Argument marshalling only: every function checks the torch tensors it is
given (device, dtype, contiguity, shape), passes their device pointers and
sizes to the C entry point of the same name on the current HIP stream, and
raises ``MLAError`` on a non-zero status.  All arithmetic runs in the HIP
kernels; there is no CPU fallback, and loading fails loudly when the library
has not been built.
"""
from __future__ import annotations

import ctypes
import heapq
import math
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_kv.so")

DTYPE_BF16 = 0
DTYPE_FP32 = 1
PAGE_SIZE = 64

EXPORTED = ("mla_absorb_q", "mla_rope_table", "mla_decode_paged", "mla_combine", "mla_up_v",
            "mla_append_kv", "mla_decode_workspace_bytes", "mla_status_string")

_lib = None


class MLAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed with status {status}: {status_string(status)}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m mla_latent_kv_09_amd.build_lib` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    P, I, F, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double
    lib.mla_absorb_q.argtypes = [P, P, P, I, I, I, I, I, I, P]
    lib.mla_rope_table.argtypes = [P, P, I, I, D, P]
    lib.mla_decode_paged.argtypes = ([P] * 8 + [I] + [P] * 2 + [I] * 12 + [F, I, I, P])
    lib.mla_combine.argtypes = [P, P, P, P, I, I, I, I, I, I, P]
    lib.mla_up_v.argtypes = [P, P, P, I, I, I, I, I, I, P]
    lib.mla_append_kv.argtypes = [P] * 8 + [I] * 9 + [P]
    lib.mla_decode_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.mla_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.mla_status_string.argtypes = [I]
    lib.mla_status_string.restype = ctypes.c_char_p
    for name in ("mla_absorb_q", "mla_rope_table", "mla_decode_paged", "mla_combine", "mla_up_v",
                 "mla_append_kv"):
        getattr(lib, name).restype = I
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().mla_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MLAError(fn, status)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_FP32
    raise TypeError(f"storage dtype must be bfloat16 or float32, got {t.dtype}")


def _dev(*ts: Optional[torch.Tensor]) -> None:
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live in GPU memory")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def absorb_q(q_c: torch.Tensor, w_uk: torch.Tensor, q_abs: Optional[torch.Tensor] = None, *,
             groups: int = 1, stream=None) -> torch.Tensor:
    """q_abs[t,h,:] = q_c[t,h,:] @ w_uk[h]; q_c [T,H,d_hc], w_uk [H,d_hc,d_c/G]."""
    T, H, d_hc = q_c.shape
    d_cg = w_uk.shape[2]
    if w_uk.shape != (H, d_hc, d_cg) or w_uk.dtype != q_c.dtype:
        raise ValueError("w_uk must be [H, d_hc, d_c/G] with q_c's dtype")
    if q_abs is None:
        q_abs = torch.empty((T, H, d_cg), dtype=q_c.dtype, device=q_c.device)
    _dev(q_c, w_uk, q_abs)
    _check("mla_absorb_q", load().mla_absorb_q(
        _ptr(q_c), _ptr(w_uk), _ptr(q_abs), T, H, groups, d_hc, d_cg * groups, _dtype_code(q_c),
        _stream(stream)))
    return q_abs


def rope_table(max_pos: int, d_R: int, base: float = 10000.0, *, device="cuda", stream=None):
    """fp32 (cos, sin) tables [max_pos, d_R/2] computed on the GPU."""
    cos = torch.empty((max_pos, d_R // 2), dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    _check("mla_rope_table", load().mla_rope_table(_ptr(cos), _ptr(sin), max_pos, d_R, float(base),
                                                   _stream(stream)))
    return cos, sin


def workspace(total_q: int, heads: int, d_cg: int, num_splits: int, device="cuda",
              dtype=torch.bfloat16):
    """Allocate the (o_part, lse_part) split workspace: o_part in the storage dtype,
    lse_part in float32."""
    o_part = torch.empty((total_q, heads, num_splits, d_cg), dtype=dtype, device=device)
    lse_part = torch.empty((total_q, heads, num_splits), dtype=torch.float32, device=device)
    return o_part, lse_part


def decode_paged(q_abs, q_r, kv_cache, page_table, seq_lens, cu_q, o_part, lse_part, *,
                 d_hc: int, groups: int = 1, rope: Optional[tuple] = None, softmax_scale: float = 0.0,
                 causal: bool = True, pages_per_split: int = 0, stream=None) -> None:
    """Split-KV attention over the paged cache into (o_part, lse_part)."""
    T, H, d_cg = q_abs.shape
    d_R = q_r.shape[2]
    P, ps, width = kv_cache.shape
    B, max_pages = page_table.shape
    S = o_part.shape[2]
    if q_r.shape[:2] != (T, H) or width != d_cg * groups + d_R:
        raise ValueError("inconsistent q_r / kv_cache shapes")
    if o_part.shape != (T, H, S, d_cg) or lse_part.shape != (T, H, S):
        raise ValueError("o_part must be [T,H,S,d_c/G] and lse_part [T,H,S]")
    for t, dt in ((page_table, torch.int32), (seq_lens, torch.int32), (cu_q, torch.int32),
                  (o_part, q_abs.dtype), (lse_part, torch.float32)):
        if t.dtype != dt:
            raise TypeError(f"expected {dt}, got {t.dtype}")
    if seq_lens.shape != (B,) or cu_q.shape != (B + 1,):
        raise ValueError("seq_lens must be [B] and cu_q [B+1]")
    if q_r.dtype != q_abs.dtype or kv_cache.dtype != q_abs.dtype:
        raise TypeError("q_abs, q_r and kv_cache must share the storage dtype")
    cos, sin = rope if rope is not None else (None, None)
    rope_max_pos = 0 if cos is None else cos.shape[0]
    _dev(q_abs, q_r, kv_cache, page_table, seq_lens, cu_q, o_part, lse_part, cos, sin)
    _check("mla_decode_paged", load().mla_decode_paged(
        _ptr(q_abs), _ptr(q_r), _ptr(kv_cache), _ptr(page_table), _ptr(seq_lens), _ptr(cu_q),
        _ptr(cos), _ptr(sin), rope_max_pos, _ptr(o_part), _ptr(lse_part),
        B, T, max_pages, P, H, groups, d_hc, d_cg * groups, d_R, ps, S, int(pages_per_split),
        float(softmax_scale),
        int(bool(causal)), _dtype_code(q_abs), _stream(stream)))


def append_kv(c_kv_new, k_r_new, kv_cache, page_table, seq_lens, cu_q, *,
              rope: Optional[tuple] = None, stream=None) -> None:
    """Write the new tokens' rows [c_KV | RoPE(k_R, pos)] into their pages of kv_cache
    (in place); c_kv_new [T, d_c], k_r_new [T, d_R], kv_cache [P, 64, d_c + d_R]."""
    T, d_c = c_kv_new.shape
    d_R = k_r_new.shape[1]
    P, ps, width = kv_cache.shape
    B, max_pages = page_table.shape
    if k_r_new.shape[0] != T or width != d_c + d_R:
        raise ValueError("inconsistent c_kv_new / k_r_new / kv_cache shapes")
    if c_kv_new.dtype != kv_cache.dtype or k_r_new.dtype != kv_cache.dtype:
        raise TypeError("c_kv_new, k_r_new and kv_cache must share the storage dtype")
    for t in (page_table, seq_lens, cu_q):
        if t.dtype != torch.int32:
            raise TypeError(f"expected int32, got {t.dtype}")
    if seq_lens.shape != (B,) or cu_q.shape != (B + 1,):
        raise ValueError("seq_lens must be [B] and cu_q [B+1]")
    cos, sin = rope if rope is not None else (None, None)
    rope_max_pos = 0 if cos is None else cos.shape[0]
    _dev(c_kv_new, k_r_new, kv_cache, page_table, seq_lens, cu_q, cos, sin)
    _check("mla_append_kv", load().mla_append_kv(
        _ptr(c_kv_new), _ptr(k_r_new), _ptr(kv_cache), _ptr(page_table), _ptr(seq_lens),
        _ptr(cu_q), _ptr(cos), _ptr(sin), rope_max_pos, B, T, max_pages, P, d_c, d_R, ps,
        _dtype_code(kv_cache), _stream(stream)))


def combine(o_part, lse_part, o_latent=None, lse_out=None, *, dtype=torch.bfloat16, stream=None):
    """LSE merge of the splits -> o_latent [T,H,d_c/G] (and optionally lse [T,H])."""
    T, H, S, d_cg = o_part.shape
    if o_latent is None:
        o_latent = torch.empty((T, H, d_cg), dtype=dtype, device=o_part.device)
    if o_part.dtype != o_latent.dtype or lse_part.dtype != torch.float32:
        raise TypeError("o_part must share o_latent's dtype and lse_part must be float32")
    _dev(o_part, lse_part, o_latent, lse_out)
    _check("mla_combine", load().mla_combine(
        _ptr(o_part), _ptr(lse_part), _ptr(o_latent), _ptr(lse_out), T, H, 1, d_cg, S,
        _dtype_code(o_latent), _stream(stream)))
    return o_latent


def up_v(o_latent, w_uv, out=None, *, groups: int = 1, stream=None):
    """out[t,h,:] = w_uv[h] @ o_latent[t,h,:]; w_uv [H,d_hc,d_c/G]."""
    T, H, d_cg = o_latent.shape
    d_hc = w_uv.shape[1]
    if w_uv.shape != (H, d_hc, d_cg) or w_uv.dtype != o_latent.dtype:
        raise ValueError("w_uv must be [H, d_hc, d_c/G] with o_latent's dtype")
    if out is None:
        out = torch.empty((T, H, d_hc), dtype=o_latent.dtype, device=o_latent.device)
    _dev(o_latent, w_uv, out)
    _check("mla_up_v", load().mla_up_v(
        _ptr(o_latent), _ptr(w_uv), _ptr(out), T, H, groups, d_hc, d_cg * groups,
        _dtype_code(o_latent), _stream(stream)))
    return out


# Cost of one split in units of one page (streaming 72 KB and computing 128 heads
# over it): a fixed part for the prologue (queries fetched, first page in flight) and
# the epilogue (bf16 partial written, 128 KB), measured at about 2.5 pages on MI355X,
# plus one unit per page.  A split with no keys exits at once.
SPLIT_OVERHEAD_PAGES = 2.5
EMPTY_SPLIT_PAGES = 0.2
XCDS = 8


def plan_makespan(pages, q_lens, pages_per_split: int, cu_count: int = 256) -> float:
    """Finish time, in page units, of the decode grid under the cost model above.  The
    grid is launched in split-fastest order (workgroup L = token * S + split); the
    dispatcher deals workgroup L to XCD L mod 8, and each XCD hands its workgroups to
    the first of its CUs to come free, one workgroup per CU at a time."""
    n_splits = max(math.ceil(p / pages_per_split) for p in pages)
    per_xcd = max(1, cu_count // XCDS)
    free = [[0.0] * per_xcd for _ in range(XCDS)]
    wg = 0
    for p, n in zip(pages, q_lens):
        for _ in range(n):
            for y in range(n_splits):
                work = min(pages_per_split, p - y * pages_per_split)
                cost = SPLIT_OVERHEAD_PAGES + work if work > 0 else EMPTY_SPLIT_PAGES
                f = free[wg % XCDS]
                heapq.heapreplace(f, f[0] + cost)
                wg += 1
    return max(max(f) for f in free)


# Longest split (pages) for which two 64-head workgroups per (token, split) pay off: the
# half-head workgroups run a page at about 0.66 of a full page's time, so twice the
# pages cost about 1.3x; in exchange the split count halves, which halves the partial
# output the decode writes and the merge reads.  Measured on 4096-key sequences at
# batch 16 (4 pages per full-head split): 58.1 against 61.4 us per step; at 1024
# pages per sequence (64 per split) the head split loses (383 against 348 us).
HEAD_SPLIT_MAX_PAGES = 6


def head_split(total_q: int, num_splits: int, groups: int, cu_count: int = 256) -> int:
    """Workgroups per (token, split) pair of the MFMA decode kernel: 2 (64 heads each)
    for one latent group when 2 * total_q * num_splits <= cu_count, else 1 (128 heads).
    The library applies the same rule to the device's compute-unit count."""
    return 2 if groups == 1 and 2 * total_q * num_splits <= cu_count else 1


def split_plan(seq_lens_host, q_lens_host, cu_count: int = 256, groups: int = 1):
    """(num_splits, pages_per_split) for a batch: the split length whose grid finishes
    first under plan_makespan's model, among at most 256 splits per sequence.  The
    candidates are the shortest split lengths for each split count of the longest
    sequence and the lengths that give k workgroups per CU for small k; a tie goes
    to the fewer workgroups (less partial output to merge).  With one latent group, a
    plan of at most HEAD_SPLIT_MAX_PAGES pages per split is then doubled in length
    when the halved split count lets the kernel run two 64-head workgroups per
    (token, split) (head_split)."""
    pages = [max(1, math.ceil(int(L) / PAGE_SIZE)) for L in seq_lens_host]
    q = [int(x) for x in q_lens_host]
    max_p = max(pages)
    total = sum(p * n for p, n in zip(pages, q))
    cands = {math.ceil(max_p / s) for s in range(1, min(256, max_p) + 1)}
    cands |= {max(1, math.ceil(total / (cu_count * k))) for k in range(1, 17)}
    cands = sorted(c for c in cands if math.ceil(max_p / c) <= 256)
    if len(cands) > 96:  # keep the evaluation cheap: the longest splits plus a spread
        cands = sorted(set(cands[-64:]) | set(cands[:: max(1, len(cands) // 32)]))
    best = None
    for pps in cands:
        n_wg = sum(n * math.ceil(p / pps) for p, n in zip(pages, q))
        key = (plan_makespan(pages, q, pps, cu_count), n_wg)
        if best is None or key < best[0]:
            best = (key, pps)
    pps = best[1]
    S = max(1, math.ceil(max_p / pps))
    if groups == 1 and S >= 2 and pps <= HEAD_SPLIT_MAX_PAGES:
        pps2 = 2 * pps
        S2 = max(1, math.ceil(max_p / pps2))
        if head_split(sum(q), S2, groups, cu_count) == 2:
            return S2, pps2
    return S, pps


class DecodeStep:
    """The four calls of one decode step over preallocated buffers (no allocation per call)."""

    def __init__(self, *, q_c, q_r, w_uk, w_uv, kv_cache, page_table, seq_lens, cu_q, groups=1,
                 num_splits=None, rope=None, causal=True, seq_lens_host=None, pages_per_split=0):
        self.q_c, self.q_r, self.w_uk, self.w_uv = q_c, q_r, w_uk, w_uv
        self.kv, self.page_table, self.seq_lens, self.cu_q = kv_cache, page_table, seq_lens, cu_q
        self.groups, self.rope, self.causal = groups, rope, causal
        T, H, d_hc = q_c.shape
        d_cg = w_uk.shape[2]
        if num_splits is None:
            lens = seq_lens_host if seq_lens_host is not None else seq_lens.cpu().tolist()
            cu = cu_q.cpu().tolist()
            num_splits, self.pages_per_split = split_plan(lens, [b - a for a, b in zip(cu, cu[1:])],
                                                          groups=groups)
        else:
            self.pages_per_split = int(pages_per_split)
        self.num_splits = num_splits
        dev = q_c.device
        self.q_abs = torch.empty((T, H, d_cg), dtype=q_c.dtype, device=dev)
        self.o_part, self.lse_part = workspace(T, H, d_cg, num_splits, dev, q_c.dtype)
        self.o_latent = torch.empty((T, H, d_cg), dtype=q_c.dtype, device=dev)
        self.lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        self.out = torch.empty((T, H, d_hc), dtype=q_c.dtype, device=dev)
        self.d_hc = d_hc

    def absorb(self, stream=None):
        absorb_q(self.q_c, self.w_uk, self.q_abs, groups=self.groups, stream=stream)

    def attend(self, stream=None):
        decode_paged(self.q_abs, self.q_r, self.kv, self.page_table, self.seq_lens, self.cu_q,
                     self.o_part, self.lse_part, d_hc=self.d_hc, groups=self.groups, rope=self.rope,
                     causal=self.causal, pages_per_split=self.pages_per_split, stream=stream)

    def merge(self, stream=None):
        combine(self.o_part, self.lse_part, self.o_latent, self.lse, stream=stream)

    def project(self, stream=None):
        up_v(self.o_latent, self.w_uv, self.out, groups=self.groups, stream=stream)

    def __call__(self, stream=None):
        self.absorb(stream)
        self.attend(stream)
        self.merge(stream)
        self.project(stream)
        return self.out
