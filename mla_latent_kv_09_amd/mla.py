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
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_kv.so")

DTYPE_BF16 = 0
DTYPE_FP32 = 1
PAGE_SIZE = 64

EXPORTED = ("mla_absorb_q", "mla_rope_table", "mla_decode_paged", "mla_combine", "mla_up_v",
            "mla_combine_up_v", "mla_combine_up_v_fused",
            "mla_append_kv", "mla_decode_workspace_bytes", "mla_decode_plan", "mla_attend_noalloc",
            "mla_decode_paged_fp8", "mla_append_kv_fp8", "mla_fp8_page_bytes",
            "mla_decode_paged_mxfp4", "mla_append_kv_mxfp4", "mla_mxfp4_page_bytes", "mla_branch",
            "mla_prefill_paged", "mla_prefill_workspace_bytes", "mla_decompress_kv",
            "mla_prefill_attention", "mla_status_string")

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
    lib.mla_combine_up_v.argtypes = [P] * 6 + [I] * 7 + [P]
    lib.mla_combine_up_v_fused.argtypes = [I] * 6
    lib.mla_combine_up_v_fused.restype = I
    lib.mla_append_kv.argtypes = [P] * 8 + [I] * 9 + [P]
    lib.mla_decode_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.mla_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.mla_decode_plan.argtypes = [P, P, I, I, I, P, P]
    lib.mla_attend_noalloc.argtypes = ([P] * 8 + [I] + [P] * 2 + [I] * 12 + [F, I, I, P])
    lib.mla_decode_paged_fp8.argtypes = ([P] * 8 + [I] + [P] * 2 + [I] * 12 + [F, I, P])
    lib.mla_append_kv_fp8.argtypes = [P] * 8 + [I] * 8 + [P]
    lib.mla_decode_paged_mxfp4.argtypes = ([P] * 8 + [I] + [P] * 2 + [I] * 12 + [F, I, P])
    lib.mla_append_kv_mxfp4.argtypes = [P] * 8 + [I] * 8 + [P]
    lib.mla_branch.argtypes = [P, I, I]
    lib.mla_prefill_paged.argtypes = [P] * 8 + [I] + [P] * 5 + [I] * 11 + [F, I, I, P]
    lib.mla_decompress_kv.argtypes = [P] * 6 + [I] * 10 + [P]
    lib.mla_prefill_attention.argtypes = [P] * 8 + [I] + [P] * 3 + [I] * 11 + [F, I, I, P]
    lib.mla_prefill_workspace_bytes.argtypes = [I, I, I, I]
    lib.mla_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.mla_fp8_page_bytes.argtypes = [I, I]
    lib.mla_fp8_page_bytes.restype = ctypes.c_size_t
    lib.mla_mxfp4_page_bytes.argtypes = [I, I]
    lib.mla_mxfp4_page_bytes.restype = ctypes.c_size_t
    lib.mla_status_string.argtypes = [I]
    lib.mla_status_string.restype = ctypes.c_char_p
    for name in ("mla_absorb_q", "mla_rope_table", "mla_decode_paged", "mla_combine", "mla_up_v",
                 "mla_combine_up_v", "mla_append_kv", "mla_decode_plan", "mla_attend_noalloc", "mla_decode_paged_fp8",
                 "mla_append_kv_fp8", "mla_decode_paged_mxfp4", "mla_append_kv_mxfp4",
                 "mla_branch", "mla_prefill_paged", "mla_decompress_kv",
                 "mla_prefill_attention"):
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


def _expect(name: str, t: Optional[torch.Tensor], shape, dtype) -> None:
    """A caller-supplied buffer must have exactly this shape and dtype."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _rope_pair(rope: Optional[tuple], d_R: int, device) -> tuple:
    """(cos, sin, max_pos) of a RoPE table pair: float32 [max_pos, d_R/2] each, on the
    device of the other tensors, or (None, None, 0) for no rotation."""
    if rope is None:
        return None, None, 0
    cos, sin = rope
    if cos is None or sin is None:
        raise ValueError("rope must be a (cos, sin) pair of tables")
    if cos.dim() != 2 or cos.shape[1] != d_R // 2 or cos.shape[0] < 1:
        raise ValueError(f"rope tables must be [max_pos, {d_R // 2}], got {tuple(cos.shape)}")
    _expect("rope sin table", sin, cos.shape, torch.float32)
    _expect("rope cos table", cos, cos.shape, torch.float32)
    if cos.device != device or sin.device != device:
        raise ValueError("rope tables must live on the device of the other tensors")
    return cos, sin, int(cos.shape[0])


def absorb_q(q_c: torch.Tensor, w_uk: torch.Tensor, q_abs: Optional[torch.Tensor] = None, *,
             groups: int = 1, stream=None) -> torch.Tensor:
    """q_abs[t,h,:] = q_c[t,h,:] @ w_uk[h]; q_c [T,H,d_hc], w_uk [H,d_hc,d_c/G]."""
    T, H, d_hc = q_c.shape
    d_cg = w_uk.shape[2]
    if w_uk.shape != (H, d_hc, d_cg) or w_uk.dtype != q_c.dtype:
        raise ValueError("w_uk must be [H, d_hc, d_c/G] with q_c's dtype")
    if q_abs is None:
        q_abs = torch.empty((T, H, d_cg), dtype=q_c.dtype, device=q_c.device)
    _expect("q_abs", q_abs, (T, H, d_cg), q_c.dtype)
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
    cos, sin, rope_max_pos = _rope_pair(rope, d_R, q_abs.device)
    _dev(q_abs, q_r, kv_cache, page_table, seq_lens, cu_q, o_part, lse_part, cos, sin)
    _check("mla_decode_paged", load().mla_decode_paged(
        _ptr(q_abs), _ptr(q_r), _ptr(kv_cache), _ptr(page_table), _ptr(seq_lens), _ptr(cu_q),
        _ptr(cos), _ptr(sin), rope_max_pos, _ptr(o_part), _ptr(lse_part),
        B, T, max_pages, P, H, groups, d_hc, d_cg * groups, d_R, ps, S, int(pages_per_split),
        float(softmax_scale),
        int(bool(causal)), _dtype_code(q_abs), _stream(stream)))


BRANCH_ABSORBED = 0
BRANCH_DECOMPRESSED = 1
PREFILL_THRESHOLD = 256


def branch(q_lens_host, threshold: int = PREFILL_THRESHOLD) -> int:
    """The library's host-only dispatch (mla_branch): BRANCH_DECOMPRESSED when the batch's
    largest query count reaches ``threshold``, else BRANCH_ABSORBED."""
    B = len(q_lens_host)
    if B == 0:
        raise ValueError("q_lens must be non-empty")
    qs = (ctypes.c_int32 * B)(*[int(x) for x in q_lens_host])
    r = load().mla_branch(qs, B, int(threshold))
    if r < 0:
        raise MLAError("mla_branch", r)
    return r


def prefill_workspace(num_pool_pages: int, heads: int, d_hc: int, device="cuda") -> torch.Tensor:
    """The decompressed branch's K/V workspace (mla_prefill_workspace_bytes bytes)."""
    n = int(load().mla_prefill_workspace_bytes(int(num_pool_pages), int(heads), int(d_hc), DTYPE_BF16))
    if n == 0:
        raise ValueError("bad sizes for the prefill workspace")
    return torch.empty(n // 2, dtype=torch.bfloat16, device=device)


def prefill_paged(q_c, q_r, kv_cache, page_table, seq_lens, cu_q, w_uk, w_uv, workspace,
                  out=None, lse_out=None, *, max_q_len: int, groups: int = 1,
                  rope: Optional[tuple] = None, softmax_scale: float = 0.0, causal: bool = True,
                  stream=None) -> torch.Tensor:
    """The decompressed branch (mla_prefill_paged): out[t,h,:] [T,H,d_hc] straight from
    q_c / q_R and the paged latent cache, K and V expanded into ``workspace``."""
    T, H, d_hc = q_c.shape
    d_R = q_r.shape[2]
    P, ps, width = kv_cache.shape
    B, max_pages = page_table.shape
    d_c = w_uk.shape[2] * groups
    if q_r.shape[:2] != (T, H) or width != d_c + d_R:
        raise ValueError("inconsistent q_r / kv_cache shapes")
    if w_uk.shape != (H, d_hc, d_c // groups) or w_uv.shape != w_uk.shape:
        raise ValueError("w_uk and w_uv must be [H, d_hc, d_c/G]")
    for t in (q_c, q_r, kv_cache, w_uk, w_uv):
        if t.dtype != torch.bfloat16:
            raise TypeError("the decompressed branch takes bf16 tensors")
    for t in (page_table, seq_lens, cu_q):
        if t.dtype != torch.int32:
            raise TypeError(f"expected int32, got {t.dtype}")
    if seq_lens.shape != (B,) or cu_q.shape != (B + 1,):
        raise ValueError("seq_lens must be [B] and cu_q [B+1]")
    need = int(load().mla_prefill_workspace_bytes(P, H, d_hc, DTYPE_BF16))
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must hold {need} bytes")
    if out is None:
        out = torch.empty((T, H, d_hc), dtype=torch.bfloat16, device=q_c.device)
    _expect("out", out, (T, H, d_hc), torch.bfloat16)
    _expect("lse_out", lse_out, (T, H), torch.float32)
    cos, sin, rope_max_pos = _rope_pair(rope, d_R, q_c.device)
    _dev(q_c, q_r, kv_cache, page_table, seq_lens, cu_q, w_uk, w_uv, workspace, out, lse_out, cos, sin)
    _check("mla_prefill_paged", load().mla_prefill_paged(
        _ptr(q_c), _ptr(q_r), _ptr(kv_cache), _ptr(page_table), _ptr(seq_lens), _ptr(cu_q),
        _ptr(cos), _ptr(sin), rope_max_pos, _ptr(w_uk), _ptr(w_uv), _ptr(workspace), _ptr(out),
        _ptr(lse_out), B, T, max_pages, P, int(max_q_len), H, groups, d_hc, d_c, d_R, ps,
        float(softmax_scale), int(bool(causal)), DTYPE_BF16, _stream(stream)))
    return out


def decompress_kv(kv_cache, page_table, seq_lens, w_uk, w_uv, workspace, *, groups: int = 1,
                  stream=None) -> None:
    """First half of the decompressed branch (mla_decompress_kv): K and V of every cache
    row of the batch into ``workspace``."""
    P, ps, width = kv_cache.shape
    B, max_pages = page_table.shape
    H, d_hc, d_cg = w_uk.shape
    d_c = d_cg * groups
    _dev(kv_cache, page_table, seq_lens, w_uk, w_uv, workspace)
    _check("mla_decompress_kv", load().mla_decompress_kv(
        _ptr(kv_cache), _ptr(page_table), _ptr(seq_lens), _ptr(w_uk), _ptr(w_uv), _ptr(workspace),
        B, max_pages, P, H, groups, d_hc, d_c, width - d_c, ps, DTYPE_BF16, _stream(stream)))


def prefill_attention(q_c, q_r, kv_cache, page_table, seq_lens, cu_q, workspace, out, lse_out=None,
                      *, max_q_len: int, d_c: int, groups: int = 1, rope: Optional[tuple] = None,
                      softmax_scale: float = 0.0, causal: bool = True, stream=None) -> None:
    """Second half of the decompressed branch (mla_prefill_attention)."""
    T, H, d_hc = q_c.shape
    d_R = q_r.shape[2]
    P, ps, width = kv_cache.shape
    B, max_pages = page_table.shape
    _expect("out", out, (T, H, d_hc), torch.bfloat16)
    _expect("lse_out", lse_out, (T, H), torch.float32)
    cos, sin, rope_max_pos = _rope_pair(rope, d_R, q_c.device)
    _dev(q_c, q_r, kv_cache, page_table, seq_lens, cu_q, workspace, out, lse_out, cos, sin)
    _check("mla_prefill_attention", load().mla_prefill_attention(
        _ptr(q_c), _ptr(q_r), _ptr(kv_cache), _ptr(page_table), _ptr(seq_lens), _ptr(cu_q),
        _ptr(cos), _ptr(sin), rope_max_pos, _ptr(workspace), _ptr(out), _ptr(lse_out),
        B, T, max_pages, P, int(max_q_len), H, groups, d_hc, d_c, d_R, ps,
        float(softmax_scale), int(bool(causal)), DTYPE_BF16, _stream(stream)))


def fp8_page_bytes(d_c: int, d_R: int) -> int:
    """Bytes of one FP8 cache page: 64 x (d_c E4M3 codes + d_R bf16 + one float32 scale)."""
    return int(load().mla_fp8_page_bytes(int(d_c), int(d_R)))


def mxfp4_page_bytes(d_c: int, d_R: int) -> int:
    """Bytes of one MXFP4 cache page: 64 x (d_c / 2 bytes of packed E2M1 codes + d_R bf16 +
    d_c / 32 E8M0 scale bytes); 0 when d_c is not a multiple of 32."""
    return int(load().mla_mxfp4_page_bytes(int(d_c), int(d_R)))


# The quantized cache formats: page bytes and the library's append and decode calls.
_QUANT = {"fp8": (fp8_page_bytes, "mla_append_kv_fp8", "mla_decode_paged_fp8"),
          "mxfp4": (mxfp4_page_bytes, "mla_append_kv_mxfp4", "mla_decode_paged_mxfp4")}


def cache_format(kv, d_c: int, d_R: int) -> str:
    """"bf16" / "fp32" for row caches, "fp8" or "mxfp4" for uint8 pages (told apart by their
    size: the two page sizes never coincide)."""
    if kv.dtype != torch.uint8:
        return "bf16" if kv.dtype == torch.bfloat16 else "fp32"
    for fmt, (page_bytes, _, _) in _QUANT.items():
        if kv.shape[1] == page_bytes(d_c, d_R):
            return fmt
    raise ValueError(f"uint8 pages of {kv.shape[1]} bytes are neither FP8 nor MXFP4 pages "
                     f"for d_c {d_c}, d_R {d_R}")


def _decode_paged_quant(fmt, q_abs, q_r, kv, page_table, seq_lens, cu_q, o_part, lse_part, *,
                        d_hc, d_R, groups, rope, softmax_scale, causal, pages_per_split, stream):
    page_bytes_fn, _, call = _QUANT[fmt]
    T, H, d_cg = q_abs.shape
    P, page_bytes = kv.shape
    B, max_pages = page_table.shape
    S = o_part.shape[2]
    d_c = d_cg * groups
    if kv.dtype != torch.uint8 or page_bytes != page_bytes_fn(d_c, d_R):
        raise ValueError(f"the {fmt} cache must be uint8 [P, {fmt}_page_bytes(d_c, d_R)]")
    if q_abs.dtype != torch.bfloat16 or q_r.dtype != torch.bfloat16:
        raise TypeError(f"the {fmt} cache decode takes bf16 queries")
    if q_r.shape != (T, H, d_R):
        raise ValueError("q_r must be [T, H, d_R]")
    _expect("o_part", o_part, (T, H, S, d_cg), torch.bfloat16)
    _expect("lse_part", lse_part, (T, H, S), torch.float32)
    for t in (page_table, seq_lens, cu_q):
        if t.dtype != torch.int32:
            raise TypeError(f"expected int32, got {t.dtype}")
    if seq_lens.shape != (B,) or cu_q.shape != (B + 1,):
        raise ValueError("seq_lens must be [B] and cu_q [B+1]")
    cos, sin, rope_max_pos = _rope_pair(rope, d_R, q_abs.device)
    _dev(q_abs, q_r, kv, page_table, seq_lens, cu_q, o_part, lse_part, cos, sin)
    _check(call, getattr(load(), call)(
        _ptr(q_abs), _ptr(q_r), _ptr(kv), _ptr(page_table), _ptr(seq_lens), _ptr(cu_q),
        _ptr(cos), _ptr(sin), rope_max_pos, _ptr(o_part), _ptr(lse_part),
        B, T, max_pages, P, H, groups, d_hc, d_c, d_R, 64, S, int(pages_per_split),
        float(softmax_scale), int(bool(causal)), _stream(stream)))


def _append_kv_quant(fmt, c_kv_new, k_r_new, kv, page_table, seq_lens, cu_q, *, rope, stream):
    page_bytes_fn, call, _ = _QUANT[fmt]
    T, d_c = c_kv_new.shape
    d_R = k_r_new.shape[1]
    P, page_bytes = kv.shape
    B, max_pages = page_table.shape
    if k_r_new.shape[0] != T or c_kv_new.dtype != torch.bfloat16 or k_r_new.dtype != torch.bfloat16:
        raise ValueError("c_kv_new [T, d_c] and k_r_new [T, d_R] must be bf16")
    if kv.dtype != torch.uint8 or page_bytes != page_bytes_fn(d_c, d_R):
        raise ValueError(f"the {fmt} cache must be uint8 [P, {fmt}_page_bytes(d_c, d_R)]")
    for t in (page_table, seq_lens, cu_q):
        if t.dtype != torch.int32:
            raise TypeError(f"expected int32, got {t.dtype}")
    if seq_lens.shape != (B,) or cu_q.shape != (B + 1,):
        raise ValueError("seq_lens must be [B] and cu_q [B+1]")
    cos, sin, rope_max_pos = _rope_pair(rope, d_R, kv.device)
    _dev(c_kv_new, k_r_new, kv, page_table, seq_lens, cu_q, cos, sin)
    _check(call, getattr(load(), call)(
        _ptr(c_kv_new), _ptr(k_r_new), _ptr(kv), _ptr(page_table), _ptr(seq_lens), _ptr(cu_q),
        _ptr(cos), _ptr(sin), rope_max_pos, B, T, max_pages, P, d_c, d_R, 64, _stream(stream)))


def decode_paged_fp8(q_abs, q_r, kv_fp8, page_table, seq_lens, cu_q, o_part, lse_part, *,
                     d_hc: int, d_R: int, groups: int = 1, rope: Optional[tuple] = None,
                     softmax_scale: float = 0.0, causal: bool = True, pages_per_split: int = 0,
                     stream=None) -> None:
    """mla_decode_paged over an FP8 cache kv_fp8 (uint8 [P, fp8_page_bytes(d_c, d_R)]):
    bf16 queries and partials, as mla_decode_paged."""
    _decode_paged_quant("fp8", q_abs, q_r, kv_fp8, page_table, seq_lens, cu_q, o_part, lse_part,
                        d_hc=d_hc, d_R=d_R, groups=groups, rope=rope, softmax_scale=softmax_scale,
                        causal=causal, pages_per_split=pages_per_split, stream=stream)


def decode_paged_mxfp4(q_abs, q_r, kv_fp4, page_table, seq_lens, cu_q, o_part, lse_part, *,
                       d_hc: int, d_R: int, groups: int = 1, rope: Optional[tuple] = None,
                       softmax_scale: float = 0.0, causal: bool = True, pages_per_split: int = 0,
                       stream=None) -> None:
    """mla_decode_paged over an MXFP4 cache kv_fp4 (uint8 [P, mxfp4_page_bytes(d_c, d_R)]):
    bf16 queries and partials, as mla_decode_paged."""
    _decode_paged_quant("mxfp4", q_abs, q_r, kv_fp4, page_table, seq_lens, cu_q, o_part, lse_part,
                        d_hc=d_hc, d_R=d_R, groups=groups, rope=rope, softmax_scale=softmax_scale,
                        causal=causal, pages_per_split=pages_per_split, stream=stream)


def append_kv_fp8(c_kv_new, k_r_new, kv_fp8, page_table, seq_lens, cu_q, *,
                  rope: Optional[tuple] = None, stream=None) -> None:
    """Quantize the new tokens' latents into the FP8 cache kv_fp8 (uint8 [P, page bytes]):
    codes and scale per token, k_R rotated at its position and kept bf16."""
    _append_kv_quant("fp8", c_kv_new, k_r_new, kv_fp8, page_table, seq_lens, cu_q, rope=rope,
                     stream=stream)


def append_kv_mxfp4(c_kv_new, k_r_new, kv_fp4, page_table, seq_lens, cu_q, *,
                    rope: Optional[tuple] = None, stream=None) -> None:
    """Quantize the new tokens' latents into the MXFP4 cache kv_fp4 (uint8 [P, page bytes]):
    packed E2M1 codes and one E8M0 scale byte per 32 elements, k_R rotated at its position
    and kept bf16."""
    _append_kv_quant("mxfp4", c_kv_new, k_r_new, kv_fp4, page_table, seq_lens, cu_q, rope=rope,
                     stream=stream)


NOALLOC_SCRATCH_BYTES = 64 << 20


def attend_noalloc(q_abs, q_r, kv_cache, page_table, seq_lens, cu_q, o_latent, lse_out=None, *,
                   d_hc: int, num_splits: int, groups: int = 1, rope: Optional[tuple] = None,
                   softmax_scale: float = 0.0, causal: bool = True, pages_per_split: int = 0,
                   stream=None) -> None:
    """mla_decode_paged followed by mla_combine, with the split partials in the library's
    static device scratch (no allocation by the library): writes o_latent [T,H,d_c/G] and,
    if given, lse_out [T,H]."""
    T, H, d_cg = q_abs.shape
    d_R = q_r.shape[2]
    P, ps, width = kv_cache.shape
    B, max_pages = page_table.shape
    if q_r.shape[:2] != (T, H) or width != d_cg * groups + d_R:
        raise ValueError("inconsistent q_r / kv_cache shapes")
    for t in (page_table, seq_lens, cu_q):
        if t.dtype != torch.int32:
            raise TypeError(f"expected int32, got {t.dtype}")
    if seq_lens.shape != (B,) or cu_q.shape != (B + 1,):
        raise ValueError("seq_lens must be [B] and cu_q [B+1]")
    if q_r.dtype != q_abs.dtype or kv_cache.dtype != q_abs.dtype:
        raise TypeError("q_abs, q_r and kv_cache must share the storage dtype")
    _expect("o_latent", o_latent, (T, H, d_cg), q_abs.dtype)
    _expect("lse_out", lse_out, (T, H), torch.float32)
    cos, sin, rope_max_pos = _rope_pair(rope, d_R, q_abs.device)
    _dev(q_abs, q_r, kv_cache, page_table, seq_lens, cu_q, o_latent, lse_out, cos, sin)
    _check("mla_attend_noalloc", load().mla_attend_noalloc(
        _ptr(q_abs), _ptr(q_r), _ptr(kv_cache), _ptr(page_table), _ptr(seq_lens), _ptr(cu_q),
        _ptr(cos), _ptr(sin), rope_max_pos, _ptr(o_latent), _ptr(lse_out),
        B, T, max_pages, P, H, groups, d_hc, d_cg * groups, d_R, ps, int(num_splits),
        int(pages_per_split), float(softmax_scale), int(bool(causal)), _dtype_code(q_abs),
        _stream(stream)))


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
    cos, sin, rope_max_pos = _rope_pair(rope, d_R, kv_cache.device)
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
    _expect("lse_part", lse_part, (T, H, S), torch.float32)
    _expect("o_latent", o_latent, (T, H, d_cg), o_part.dtype)
    _expect("lse_out", lse_out, (T, H), torch.float32)
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
    _expect("out", out, (T, H, d_hc), o_latent.dtype)
    _dev(o_latent, w_uv, out)
    _check("mla_up_v", load().mla_up_v(
        _ptr(o_latent), _ptr(w_uv), _ptr(out), T, H, groups, d_hc, d_cg * groups,
        _dtype_code(o_latent), _stream(stream)))
    return out


def combine_up_v_fused(heads: int, groups: int, d_hc: int, d_c: int, num_splits: int,
                       dtype=torch.bfloat16) -> bool:
    """Whether mla_combine_up_v runs this shape as one launch (host only)."""
    code = DTYPE_BF16 if dtype == torch.bfloat16 else DTYPE_FP32
    return bool(load().mla_combine_up_v_fused(heads, groups, d_hc, d_c, num_splits, code))


def combine_up_v(o_part, lse_part, w_uv, out=None, *, o_latent=None, lse_out=None, groups: int = 1,
                 stream=None):
    """combine then up_v in one call (one launch where the fused kernel covers the shape;
    o_latent, if given, receives the merged rows and is required otherwise)."""
    T, H, S, d_cg = o_part.shape
    d_hc = w_uv.shape[1]
    if w_uv.shape != (H, d_hc, d_cg) or w_uv.dtype != o_part.dtype or lse_part.dtype != torch.float32:
        raise ValueError("w_uv must be [H, d_hc, d_c/G] with o_part's dtype; lse_part float32")
    if out is None:
        out = torch.empty((T, H, d_hc), dtype=o_part.dtype, device=o_part.device)
    _expect("lse_part", lse_part, (T, H, S), torch.float32)
    _expect("o_latent", o_latent, (T, H, d_cg), o_part.dtype)
    _expect("out", out, (T, H, d_hc), o_part.dtype)
    _expect("lse_out", lse_out, (T, H), torch.float32)
    _dev(o_part, lse_part, w_uv, out, o_latent, lse_out)
    _check("mla_combine_up_v", load().mla_combine_up_v(
        _ptr(o_part), _ptr(lse_part), _ptr(w_uv), _ptr(o_latent), _ptr(out), _ptr(lse_out), T, H,
        groups, d_hc, d_cg * groups, S, _dtype_code(o_part), _stream(stream)))
    return out


def split_plan(seq_lens_host, q_lens_host, cu_count: int = 256, groups: int = 1):
    """(num_splits, pages_per_split) for a batch, from the library's host-only planner
    ``mla_decode_plan`` (host lists or arrays of int; no GPU is touched)."""
    B = len(seq_lens_host)
    if B == 0 or len(q_lens_host) != B:
        raise ValueError("seq_lens and q_lens must be non-empty and of equal length")
    lens = (ctypes.c_int32 * B)(*[int(x) for x in seq_lens_host])
    qs = (ctypes.c_int32 * B)(*[int(x) for x in q_lens_host])
    S, pps = ctypes.c_int(0), ctypes.c_int(0)
    _check("mla_decode_plan", load().mla_decode_plan(lens, qs, B, int(groups), int(cu_count),
                                                     ctypes.byref(S), ctypes.byref(pps)))
    return S.value, pps.value


class DecodeStep:
    """The four calls of one decode step over preallocated buffers (no allocation per call)."""

    def __init__(self, *, q_c, q_r, w_uk, w_uv, kv_cache, page_table, seq_lens, cu_q, groups=1,
                 num_splits=None, rope=None, causal=True, seq_lens_host=None, pages_per_split=0,
                 threshold=None, keep_latent=True):
        self.q_c, self.q_r, self.w_uk, self.w_uv = q_c, q_r, w_uk, w_uv
        self.kv, self.page_table, self.seq_lens, self.cu_q = kv_cache, page_table, seq_lens, cu_q
        self.groups, self.rope, self.causal = groups, rope, causal
        self.fused = False
        # keep_latent: the merged rows (self.o_latent) are written even when the merge and
        # W_UV run as one launch (they are the two-call path's intermediate anyway)
        self.keep_latent = keep_latent
        T, H, d_hc = q_c.shape
        d_cg = w_uk.shape[2]
        cu = cu_q.cpu().tolist()
        q_lens = [b - a for a, b in zip(cu, cu[1:])]
        self.max_q_len = max(q_lens) if q_lens else 0
        # threshold None: always the absorbed calls; else the library's dispatch decides.
        self.branch = (BRANCH_ABSORBED if threshold is None or T == 0
                       else branch(q_lens, threshold))
        if self.branch == BRANCH_DECOMPRESSED:
            self.workspace = prefill_workspace(kv_cache.shape[0], H, d_hc, q_c.device)
        dev = q_c.device
        if self.branch == BRANCH_DECOMPRESSED:  # the absorbed calls' buffers are not needed
            self.num_splits, self.pages_per_split = 0, 0
        else:
            if num_splits is None:
                lens = seq_lens_host if seq_lens_host is not None else seq_lens.cpu().tolist()
                cus = torch.cuda.get_device_properties(q_c.device).multi_processor_count
                num_splits, self.pages_per_split = split_plan(lens, q_lens, cu_count=cus, groups=groups)
            else:
                self.pages_per_split = int(pages_per_split)
            self.num_splits = num_splits
            self.q_abs = torch.empty((T, H, d_cg), dtype=q_c.dtype, device=dev)
            self.o_part, self.lse_part = workspace(T, H, d_cg, num_splits, dev, q_c.dtype)
            self.o_latent = torch.empty((T, H, d_cg), dtype=q_c.dtype, device=dev)
            # merge and W_UV in one launch where the fused kernel covers the shape
            self.fused = combine_up_v_fused(H, groups, d_hc, d_cg * groups, num_splits, q_c.dtype)
        self.lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        self.out = torch.empty((T, H, d_hc), dtype=q_c.dtype, device=dev)
        self.d_hc = d_hc

    def absorb(self, stream=None):
        absorb_q(self.q_c, self.w_uk, self.q_abs, groups=self.groups, stream=stream)

    def attend(self, stream=None):
        if self.kv.dtype == torch.uint8:  # FP8 or MXFP4 cache pages
            d_R = self.q_r.shape[2]
            fmt = cache_format(self.kv, self.q_abs.shape[2] * self.groups, d_R)
            _decode_paged_quant(fmt, self.q_abs, self.q_r, self.kv, self.page_table, self.seq_lens,
                                self.cu_q, self.o_part, self.lse_part, d_hc=self.d_hc, d_R=d_R,
                                groups=self.groups, rope=self.rope, softmax_scale=0.0,
                                causal=self.causal, pages_per_split=self.pages_per_split,
                                stream=stream)
            return
        decode_paged(self.q_abs, self.q_r, self.kv, self.page_table, self.seq_lens, self.cu_q,
                     self.o_part, self.lse_part, d_hc=self.d_hc, groups=self.groups, rope=self.rope,
                     causal=self.causal, pages_per_split=self.pages_per_split, stream=stream)

    def merge(self, stream=None):
        combine(self.o_part, self.lse_part, self.o_latent, self.lse, stream=stream)

    def project(self, stream=None):
        up_v(self.o_latent, self.w_uv, self.out, groups=self.groups, stream=stream)

    def merge_project(self, stream=None):
        """merge then project: one launch when self.fused (the merged rows stay on chip)."""
        combine_up_v(self.o_part, self.lse_part, self.w_uv, self.out,
                     o_latent=None if self.fused and not self.keep_latent else self.o_latent,
                     lse_out=self.lse,
                     groups=self.groups, stream=stream)

    def prefill(self, stream=None):
        prefill_paged(self.q_c, self.q_r, self.kv, self.page_table, self.seq_lens, self.cu_q,
                      self.w_uk, self.w_uv, self.workspace, self.out, self.lse,
                      max_q_len=self.max_q_len, groups=self.groups, rope=self.rope,
                      causal=self.causal, stream=stream)

    def decompress(self, stream=None):
        decompress_kv(self.kv, self.page_table, self.seq_lens, self.w_uk, self.w_uv, self.workspace,
                      groups=self.groups, stream=stream)

    def prefill_attend(self, stream=None):
        prefill_attention(self.q_c, self.q_r, self.kv, self.page_table, self.seq_lens, self.cu_q,
                          self.workspace, self.out, self.lse, max_q_len=self.max_q_len,
                          d_c=self.w_uk.shape[2] * self.groups, groups=self.groups, rope=self.rope,
                          causal=self.causal, stream=stream)

    def __call__(self, stream=None):
        if self.branch == BRANCH_DECOMPRESSED:
            self.prefill(stream)
            return self.out
        self.absorb(stream)
        self.attend(stream)
        self.merge_project(stream)
        return self.out
