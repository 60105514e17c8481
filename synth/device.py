"""Copy a synthetic workload to device tensors (plumbing only; no arithmetic)."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass
class DeviceWorkload:
    rg: object            # sparse_decode_attention_csa2_amd.Ragged
    idx_k: torch.Tensor
    main_kv: torch.Tensor
    blk_sum: torch.Tensor
    swa: torch.Tensor
    swa_scale: torch.Tensor
    q: torch.Tensor
    q_idx: torch.Tensor
    w: torch.Tensor

    def decode_inputs(self):
        return (self.rg, self.idx_k, self.main_kv, self.blk_sum, self.swa, self.swa_scale, self.q, self.q_idx,
                self.w)


def _t(a: np.ndarray, dev, dtype=None) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    t = torch.from_numpy(a)
    if t.numel() == 0:
        t = torch.zeros(max(1, t.numel()), dtype=t.dtype)
    return t.to(dev, dtype=dtype) if dtype is not None else t.to(dev)


def upload(wl, device="cuda") -> DeviceWorkload:
    from sparse_decode_attention_csa2_amd import Ragged
    dev = torch.device(device)
    rows_per = np.diff(wl.row_off)
    paged = getattr(wl, "page_table", None) is not None
    row_len = getattr(wl, "row_len", None)
    rg = Ragged(entry_off=_t(wl.entry_off, dev), block_off=None if paged else _t(wl.block_off, dev),
                row_off=_t(wl.row_off, dev), row_req=_t(wl.row_req, dev), row_swa_start=_t(wl.row_swa_start, dev),
                row_swa_len=_t(wl.row_swa_len, dev), max_entries=wl.max_entries,
                total_entries=int(wl.idx_k.shape[0]), total_blocks=int(wl.blk_sum.shape[0]),
                swa_tokens=int(wl.swa_off[-1]), max_rows_per_request=int(rows_per.max()) if rows_per.size else 1,
                row_len=None if row_len is None else _t(np.asarray(row_len, dtype=np.int64), dev),
                page_table=_t(wl.page_table, dev) if paged else None,
                total_pages=int(wl.total_pages) if paged else 0)
    return DeviceWorkload(rg=rg, idx_k=_t(wl.idx_k, dev), main_kv=_t(wl.main_kv, dev), blk_sum=_t(wl.blk_sum, dev),
                          swa=_t(wl.swa, dev), swa_scale=_t(wl.swa_scale, dev), q=_t(wl.q, dev),
                          q_idx=_t(wl.q_idx, dev), w=_t(wl.w, dev))
