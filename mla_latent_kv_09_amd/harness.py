"""Move a generated workload into GPU memory and wire up one decode step.

Marshalling only: numpy host arrays become torch device tensors of the
storage dtype; the decode step itself is ``mla.DecodeStep`` (the four C-ABI
calls).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import mla
from .workloads import NewTokens, Workload


@dataclass
class DeviceWorkload:
    q_c: torch.Tensor
    q_r: torch.Tensor
    w_uk: torch.Tensor
    w_uv: torch.Tensor
    kv: torch.Tensor
    page_table: torch.Tensor
    seq_lens: torch.Tensor
    cu_q: torch.Tensor
    rope: Optional[tuple]


def _storage_tensor(w: Workload, x: np.ndarray, device) -> torch.Tensor:
    if w.cfg.dtype == "bf16":
        bits = x if x.dtype == np.uint16 else w.storage(x)
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def to_device(w: Workload, device="cuda", *, rope: bool = True,
              kv: Optional[np.ndarray] = None) -> DeviceWorkload:
    """Copy ``w`` to ``device``; with ``rope`` the fp32 table is built there by the library.
    ``kv`` replaces the workload's bf16 pool (an FP8 or MXFP4 pool: uint8 [P, page bytes])."""
    dev = torch.device(device)
    table = None
    if rope and w.cfg.rope_base is not None:
        max_pos = max(1, int(w.seq_lens.max()))
        table = mla.rope_table(max_pos, w.cfg.d_R, w.cfg.rope_base, device=dev)
    return DeviceWorkload(
        q_c=_storage_tensor(w, w.q_c, dev),
        q_r=_storage_tensor(w, w.q_r, dev),
        w_uk=_storage_tensor(w, w.w_uk, dev),
        w_uv=_storage_tensor(w, w.w_uv, dev),
        kv=_storage_tensor(w, w.pool, dev) if kv is None else torch.from_numpy(kv).to(dev),
        page_table=torch.from_numpy(w.page_table).to(dev),
        seq_lens=torch.from_numpy(w.seq_lens).to(dev),
        cu_q=torch.from_numpy(w.cu_q).to(dev),
        rope=table,
    )


def make_step(w: Workload, d: DeviceWorkload, num_splits: Optional[int] = None,
              pages_per_split: int = 0, threshold: Optional[int] = None,
              keep_latent: bool = True) -> mla.DecodeStep:
    """The step over `d`: the planner's split plan, or num_splits splits of
    pages_per_split pages each (0: each sequence cut into num_splits equal parts).  With a
    threshold the library's dispatch picks the absorbed calls or the decompressed branch.
    keep_latent=False lets a fused merge launch skip writing the merged rows."""
    return mla.DecodeStep(q_c=d.q_c, q_r=d.q_r, w_uk=d.w_uk, w_uv=d.w_uv, kv_cache=d.kv,
                          page_table=d.page_table, seq_lens=d.seq_lens, cu_q=d.cu_q,
                          groups=w.cfg.groups, num_splits=num_splits, rope=d.rope,
                          causal=w.cfg.causal, seq_lens_host=w.seq_lens.tolist(),
                          pages_per_split=pages_per_split, threshold=threshold,
                          keep_latent=keep_latent)


def new_tokens_to_device(w: Workload, new: NewTokens, device="cuda"):
    """(c_kv_new, k_r_new) device tensors of the storage dtype for ``mla.append_kv``."""
    dev = torch.device(device)
    return _storage_tensor(w, new.c_kv, dev), _storage_tensor(w, new.k_r, dev)


def quant_pool_by_append(w: Workload, d: DeviceWorkload, fmt: str = "fp8") -> torch.Tensor:
    """A quantized cache ("fp8" or "mxfp4") holding ``w``'s sequences, written by the
    library's append for that format from the bf16 rows already on the device: every
    sequence appended whole from position 0, k_R copied unrotated (it is stored rotated
    already).  Unused slots hold 0xFF bytes (FP8: NaN codes, NaN k_R, NaN scales; MXFP4:
    codes -6, NaN k_R, the out-of-format scale byte 255)."""
    cfg = w.cfg
    ps = cfg.page_size
    lens = [int(L) for L in w.seq_lens]
    idx = np.concatenate([
        w.page_table[b, np.arange(L) // ps].astype(np.int64) * ps + np.arange(L) % ps
        for b, L in enumerate(lens) if L > 0] or [np.zeros(0, np.int64)])
    rows = d.kv.view(-1, cfg.row)[torch.from_numpy(idx).to(d.kv.device)]
    c = rows[:, :cfg.d_c].contiguous()
    k = rows[:, cfg.d_c:].contiguous()
    P = w.num_pool_pages
    page_bytes = mla.fp8_page_bytes if fmt == "fp8" else mla.mxfp4_page_bytes
    kvq = torch.full((P, page_bytes(cfg.d_c, cfg.d_R)), 0xFF, dtype=torch.uint8, device=d.kv.device)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(d.kv.device)
    append = mla.append_kv_fp8 if fmt == "fp8" else mla.append_kv_mxfp4
    append(c, k, kvq, d.page_table, d.seq_lens, cu)
    return kvq


def fp8_pool_by_append(w: Workload, d: DeviceWorkload) -> torch.Tensor:
    """quant_pool_by_append for the FP8 cache."""
    return quant_pool_by_append(w, d, "fp8")
