"""Helpers for the GPU tests: build a device pool from a workload, run the projection through the
C-ABI, and compute the oracle's answer for the same inputs."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import rank_gemm_unified_amd as rg
from workloads import Workload, storage_to_f64


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dtype_code(w: Workload) -> int:
    return rg.LORA_F32 if w.dtype == "f32" else rg.LORA_BF16


def device_pool(w: Workload, stream=None) -> rg.Pool:
    pool = rg.Pool(w.num_pages, w.hidden, dtype_code(w), n_slots=w.n_slots, max_adapters=w.max_adapters,
                   max_rank=w.max_rank, free_order=w.free_order)
    st = pool.run_ops(w.ops, w.ranks, w.adapter, stream)
    assert all(s == 0 for s in st), (st, rg.lora_last_error())
    return pool


def ids_ranks_scale(w: Workload, ids=None):
    ids = w.ids if ids is None else ids
    d = torch.device("cuda")
    return (torch.as_tensor(np.ascontiguousarray(ids, np.int32), device=d),
            torch.as_tensor(w.ranks, device=d), torch.as_tensor(w.scales, device=d))


def run(pool: rg.Pool, w: Workload, slot: int, ids=None, x=None, stream=None) -> torch.Tensor:
    x = w.x_for_slot(slot) if x is None else x
    d_ids, d_ranks, d_scale = ids_ranks_scale(w, ids)
    y = torch.empty_like(x)
    pool.project(slot, x, w.W(slot), d_ids, d_ranks, d_scale, y=y, stream=stream)
    return y


def oracle_y(w: Workload, slot: int, rows=None, ids=None, x=None) -> np.ndarray:
    """fp64 oracle for the given rows (all by default) of one slot."""
    ids = w.ids if ids is None else np.asarray(ids)
    x = w.x_for_slot(slot) if x is None else x
    rows = np.arange(ids.size) if rows is None else np.asarray(rows)
    x64 = storage_to_f64(x[torch.as_tensor(rows, device=x.device)])
    W64 = storage_to_f64(w.W(slot)).T                    # out-major storage -> W[k, n]
    A, B = {}, {}
    for a in np.unique(ids[rows]):
        a = int(a)
        if a < 0 or int(w.ranks[a]) == 0:
            continue
        at, b = w.adapter(a)
        A[a] = storage_to_f64(at[slot]).T
        B[a] = storage_to_f64(b[slot])
    return oracle.project(x64, W64, A, B, ids[rows], w.scales)


def errors(y_gpu: torch.Tensor, y_ref: np.ndarray):
    g = storage_to_f64(y_gpu)
    rel = float(np.linalg.norm(g - y_ref) / max(np.linalg.norm(y_ref), 1e-300))
    mx = float(np.max(np.abs(g - y_ref))) if g.size else 0.0
    return rel, mx


def bf16_round_f64(y: np.ndarray) -> torch.Tensor:
    """Round exactly-representable-in-f32 values to bfloat16 (single rounding)."""
    return torch.as_tensor(y.astype(np.float32)).to(torch.bfloat16)
