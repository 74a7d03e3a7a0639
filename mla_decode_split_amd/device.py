"""Device-side buffers for a decode batch (argument marshalling only).

Moves the host arrays of a batch to HIP device memory through torch, allocates
the output and the workspace a plan asks for, and calls mla_decode_run.  No
arithmetic of the decode happens here.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import (Plan, make_problem, mla_decode_merge, mla_decode_plan, mla_decode_plan_describe, mla_decode_run,
               mla_decode_run_paged, mla_decode_split, mla_decode_split_paged, mla_plan_options)


@dataclass
class DeviceBatch:
    q: torch.Tensor
    q_scale: torch.Tensor | None
    kv: torch.Tensor
    kv_scale: torch.Tensor | None
    qo_indptr: torch.Tensor
    kv_indptr: torch.Tensor
    kv_indptr_host: np.ndarray
    max_q_len: int
    logit_cap: float
    kv_indices: torch.Tensor | None  # paged KV (page size 1): CSR row j is kv row kv_indices[j]
    kv_page_indptr: torch.Tensor | None  # pages of page_size > 1 rows: sequence b's page list start
    page_size: int                   # paged KV: rows per page
    total_kv_rows: int               # CSR rows (kv rows when not paged)
    q_dtype: str
    kv_dtype: str
    sm_scale: float

    @property
    def batch_size(self) -> int:
        return int(self.kv_indptr.shape[0] - 1)

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def total_kv(self) -> int:
        return self.total_kv_rows

    @property
    def kv_rows(self) -> int:
        return int(self.kv.shape[0])


def _to_dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def upload(w, device="cuda") -> DeviceBatch:
    """Copy a ``synth.Workload``-like object (numpy byte arrays) to the device."""
    q = _to_dev(w.q.view(np.uint8) if w.q.dtype != np.uint8 else w.q, device)
    kv = _to_dev(w.kv.view(np.uint8) if w.kv.dtype != np.uint8 else w.kv, device)
    q_scale = None if w.q_scale is None else torch.tensor([float(w.q_scale)], dtype=torch.float32, device=device)
    if w.kv_dtype == "fp8":
        kv_scale = torch.tensor([float(w.kv_scale)], dtype=torch.float32, device=device)
    elif w.kv_dtype == "mxfp4":
        # scale rows are read in 16-byte units: pad the allocation to a multiple of 16 bytes
        flat = np.ascontiguousarray(w.kv_scale, dtype=np.uint8).reshape(-1)
        pad = np.zeros((-flat.size) % 16 + 16, dtype=np.uint8)
        kv_scale = _to_dev(np.concatenate([flat, pad]), device)
    else:
        kv_scale = None
    return DeviceBatch(q=q, q_scale=q_scale, kv=kv, kv_scale=kv_scale,
                       qo_indptr=_to_dev(w.qo_indptr.astype(np.int32), device),
                       kv_indptr=_to_dev(w.kv_indptr.astype(np.int32), device),
                       kv_indptr_host=np.ascontiguousarray(w.kv_indptr, dtype=np.int32),
                       max_q_len=int(np.diff(np.asarray(w.qo_indptr, dtype=np.int64)).max(initial=0)),
                       logit_cap=float(getattr(w, "logit_cap", 0.0)),
                       kv_indices=None if getattr(w, "kv_indices", None) is None
                       else _to_dev(np.asarray(w.kv_indices, dtype=np.int32), device),
                       kv_page_indptr=None if getattr(w, "kv_page_indptr", None) is None
                       else _to_dev(np.asarray(w.kv_page_indptr, dtype=np.int32), device),
                       page_size=int(getattr(w, "page_size", 1)),
                       total_kv_rows=int(w.total_kv),
                       q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, sm_scale=float(w.sm_scale))


def plan_for(batch: DeviceBatch, rows_per_split: int = 0, wgs_per_cu: int = 0, use_host_indptr: bool = True,
             num_cus: int = 0, age_skew: int = 0, xcd_group: int = 0) -> Plan:
    prob = make_problem(batch.batch_size, batch.total_kv, batch.q_dtype, batch.kv_dtype, total_q=batch.total_q,
                        sm_scale=batch.sm_scale, num_cus=num_cus, max_q_len=batch.max_q_len,
                        logit_cap=batch.logit_cap, kv_paged=batch.page_size if batch.kv_indices is not None else 0)
    fields = (rows_per_split, wgs_per_cu, age_skew, xcd_group)
    opts = mla_plan_options(*fields) if any(fields) else None
    return mla_decode_plan(prob, opts, batch.kv_indptr_host if use_host_indptr else None)


def workspace_for(plan: Plan, device="cuda", fill: float | None = None) -> torch.Tensor:
    n = max(plan.workspace_bytes, 256)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    if fill is not None:
        ws.view(torch.float32)[: n // 4].fill_(fill)
    return ws


def run(plan: Plan, batch: DeviceBatch, out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
        stream=None) -> torch.Tensor:
    if out is None:
        out = torch.empty((batch.total_q, 16, 512), dtype=torch.bfloat16, device=batch.q.device)
    if workspace is None:
        workspace = workspace_for(plan, batch.q.device)
    if batch.kv_indices is not None:
        mla_decode_run_paged(plan, batch.q, batch.q_scale, batch.kv, batch.kv_scale, batch.kv_rows, batch.kv_indices,
                             batch.kv_page_indptr, batch.qo_indptr, batch.kv_indptr, out, workspace, workspace.numel(),
                             stream)
    else:
        mla_decode_run(plan, batch.q, batch.q_scale, batch.kv, batch.kv_scale, batch.qo_indptr, batch.kv_indptr, out,
                       workspace, workspace.numel(), stream)
    return out


def run_split(plan: Plan, batch: DeviceBatch, out: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    if batch.kv_indices is not None:
        mla_decode_split_paged(plan, batch.q, batch.q_scale, batch.kv, batch.kv_scale, batch.kv_rows,
                               batch.kv_indices, batch.kv_page_indptr, batch.qo_indptr, batch.kv_indptr, out,
                               workspace, workspace.numel(), stream)
    else:
        mla_decode_split(plan, batch.q, batch.q_scale, batch.kv, batch.kv_scale, batch.qo_indptr, batch.kv_indptr,
                         out, workspace, workspace.numel(), stream)


def run_merge(plan: Plan, batch: DeviceBatch, out: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    mla_decode_merge(plan, batch.qo_indptr, batch.kv_indptr, out, workspace, workspace.numel(), stream)


__all__ = ["run_split", "run_merge", "DeviceBatch", "upload", "plan_for", "workspace_for", "run", "mla_decode_plan_describe"]
