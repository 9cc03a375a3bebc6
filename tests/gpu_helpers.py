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


def within_one_rounding(y: torch.Tensor, y_other: torch.Tensor, floor: float = 1e-5) -> bool:
    """Two bfloat16 results of the same sums taken in different float32 orders (another split of K):
    equal up to one bfloat16 step at the larger magnitude, plus a small absolute floor for the
    float32 order difference near zero."""
    a, b = y.float(), y_other.float()
    m = torch.maximum(a.abs(), b.abs())
    ulp = torch.where(m > 0, torch.exp2(torch.floor(torch.log2(m)) - 7), torch.zeros_like(m))
    return bool(((a - b).abs() <= ulp + floor).all())


def bf16_round_f64(y: np.ndarray) -> torch.Tensor:
    """Round exactly-representable-in-f32 values to bfloat16 (single rounding)."""
    return torch.as_tensor(y.astype(np.float32)).to(torch.bfloat16)


def check_grouping(order: np.ndarray, ids: np.ndarray, ranks: np.ndarray, decode: bool) -> None:
    """The token grouping the kernels consumed (lora_debug_project's order_out) is valid: its first n
    positions hold exactly the n tokens with a low-rank term, each once and with its own adapter, and
    each adapter's tokens form one contiguous run.  Decode path: runs ordered by the quarter count of
    the rank, ceil(r / 16), from 4 down to 1, then by first token; then every other token with
    adapter -1.  Prefill path: runs in adapter order, the rest untouched (-1)."""
    ids = np.asarray(ids)
    live = np.array([a >= 0 and int(ranks[a]) > 0 for a in ids], bool)
    n = int(live.sum())
    toks, ads = order[:, 0], order[:, 1]
    assert np.array_equal(np.sort(toks[:n]), np.nonzero(live)[0]), "grouped tokens are not the adapter tokens"
    assert np.array_equal(ads[:n], ids[toks[:n]]), "a token sits in another adapter's segment"
    runs = [int(a) for i, a in enumerate(ads[:n]) if i == 0 or a != ads[i - 1]]
    assert len(runs) == len(set(runs)), "an adapter's tokens are split over several runs"
    if decode:
        first = {}
        for t, a in enumerate(ids):
            if live[t]:
                first.setdefault(int(a), t)
        assert runs == sorted(first, key=lambda a: (-((int(ranks[a]) + 15) // 16), first[a])), \
            "segments not ordered by rank quarters, then first token"
        assert np.array_equal(np.sort(toks[n:]), np.nonzero(~live)[0]) and (ads[n:] == -1).all()
    else:
        assert runs == sorted(runs), "segments not in adapter order"
        assert (order[n:] == -1).all()


def check_indices(pool: rg.Pool, w: Workload, slot: int, ids=None, x=None) -> dict:
    """Bit-exact check of the projection's own indices: lora_debug_project runs the production kernels
    (their debug instantiations) and reports, per token, the pages they multiplied in and the grouping
    they consumed.  Checks: y equals lora_project's bit for bit; the pages equal the oracle's table
    lookup (oracle.gather_page_ids) bit for bit; the grouping is valid (check_grouping)."""
    ids = np.asarray(w.ids if ids is None else ids, np.int32)
    x = w.x_for_slot(slot) if x is None else x
    T = int(ids.size)
    d_ids, d_ranks, d_scale = ids_ranks_scale(w, ids)
    y_ref = torch.empty_like(x)
    pool.project(slot, x, w.W(slot), d_ids, d_ranks, d_scale, y=y_ref)
    y = torch.empty_like(x)
    R2 = 2 * w.max_rank
    g = torch.empty((T, R2), dtype=torch.int32, device=x.device)
    o = torch.empty((T, 2), dtype=torch.int32, device=x.device)
    rg.lora_debug_project(pool.handle, x, w.W(slot), pool.table[slot], d_ids, d_ranks, d_scale, T, y,
                          pool.workspace(T), g, o)
    torch.cuda.synchronize()
    assert rg.lora_check_device_errors(pool.handle, check=False) == 0, rg.lora_last_error()
    bits = (lambda t: t.view(torch.int16)) if y.dtype == torch.bfloat16 else (lambda t: t.view(torch.int32))
    assert torch.equal(bits(y), bits(y_ref)), "debug instantiation changed y"
    want = oracle.gather_page_ids(pool.table[slot].cpu().numpy(), ids, w.ranks, w.max_rank)
    got = g.cpu().numpy()
    bad = np.nonzero((got != want).any(axis=1))[0]
    assert bad.size == 0, {"tokens": bad[:8].tolist(), "ids": ids[bad[:8]].tolist(),
                           "got": got[bad[0]].tolist(), "want": want[bad[0]].tolist()}
    check_grouping(o.cpu().numpy(), ids, w.ranks, decode=(w.dtype == "bf16" and T <= 256))
    live = sum(1 for a in ids if a >= 0 and int(w.ranks[a]) > 0)
    return {"tokens": T, "with_adapter": live, "pages_checked": int((want >= 0).sum())}
