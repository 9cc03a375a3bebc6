"""Seeded generators for the five synthetic workloads and for small test cases.

Every random value is drawn in float32 from a torch generator seeded from
``numpy.random.SeedSequence([master, kind, index...])`` and then rounded once to the storage type
(round-to-nearest-even for bfloat16).  Those rounded values *are* the inputs: the oracle widens
them exactly to float64, the HIP path reads their bits.

Integer draws (adapter ids, ranks, page placement, pool operations) use numpy generators spawned
from the same master seed.  Nothing here multiplies or adds inputs together.

Layouts (what the library's entry points expect):
  x        [T][H]                        row-major, storage dtype
  W        [H_out][H_in]  = W^T          out-major, the layout of a linear layer's weight
  A_t      [n_slots][r][H]  = A^T        row j is column j of A: one pool page
  B        [n_slots][r][H]               row j of B: one pool page
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

CONFIG_NAMES = ("tiny", "decode", "prefill", "many", "stack13b")
MAX_RANK = 64

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
_ELEM = {"f32": 4, "bf16": 2}

# master seeds, one per named workload
_MASTER = {"tiny": 101, "decode": 102, "prefill": 103, "many": 104, "stack13b": 105}
# kind codes mixed into the seed sequence
_K_W, _K_AB, _K_X, _K_IDS, _K_RANKS, _K_POOL, _K_CANARY = range(7)


def _seed(master: int, *key: int) -> int:
    return int(np.random.SeedSequence([master, *key]).generate_state(1, np.uint64)[0] >> np.uint64(1))


def _rng(master: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([master, *key]))


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bfloat16 bit patterns, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def storage_to_f64(t) -> np.ndarray:
    """Exact widening of a float32/bfloat16 tensor (any device) or array to a float64 ndarray."""
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def _draw(shape, std: float, seed: int, dtype: str, device, values: str) -> torch.Tensor:
    g = torch.Generator(device=device).manual_seed(seed)
    if values == "normal":
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
    elif values == "int":  # entries in {-1, 0, 1}
        t = torch.randint(-1, 2, shape, generator=g, device=device).to(torch.float32)
    else:
        raise ValueError(values)
    return t.to(_DT[dtype]).contiguous()


def _finite_zipf(rng: np.random.Generator, n: int, alpha: float, size: int) -> np.ndarray:
    """P(k) proportional to k^-alpha for k = 1..n; returns k-1 (adapter index)."""
    w = np.arange(1, n + 1, dtype=np.float64) ** (-alpha)
    return rng.choice(n, size=size, p=w / w.sum()).astype(np.int32)


@dataclass
class Workload:
    """One synthetic multi-LoRA workload.  Tensors are drawn lazily and cached."""

    name: str
    hidden: int
    dtype: str                      # "f32" | "bf16"
    n_slots: int                    # (layer, projection) pairs, each with its own W, A, B
    max_adapters: int
    T: int
    ids: np.ndarray                 # int32 [T], -1 = no adapter
    ranks: np.ndarray               # int32 [max_adapters]
    scales: np.ndarray              # float32 [max_adapters]
    slot_x: list                    # slot -> index of the x it reads
    n_x: int
    num_pages: int
    free_order: np.ndarray          # int64 [num_pages]: initial free list (popped from the end)
    ops: list                       # pool operations, executed in order (see pool_ops doc)
    master: int
    device: str = "cpu"
    values: str = "normal"          # "normal" | "int"
    w_std: float = 0.02
    ab_std: float = 0.02
    x_std: float = 1.0
    max_rank: int = MAX_RANK
    segments: list = field(default_factory=list)   # prefill runs (start, length) if any
    _cache: dict = field(default_factory=dict, repr=False)

    # ---- sizes -------------------------------------------------------------------------
    @property
    def elem(self) -> int:
        return _ELEM[self.dtype]

    @property
    def torch_dtype(self):
        return _DT[self.dtype]

    def loaded_adapters(self) -> list:
        out = []
        for op in self.ops:
            if op[0] == "load" and op[1] not in out:
                out.append(op[1])
        return out

    # ---- tensors -----------------------------------------------------------------------
    def x(self, i: int = 0) -> torch.Tensor:
        key = ("x", i)
        if key not in self._cache:
            self._cache[key] = _draw((self.T, self.hidden), self.x_std,
                                     _seed(self.master, _K_X, i), self.dtype, self.device, self.values)
        return self._cache[key]

    def x_for_slot(self, slot: int) -> torch.Tensor:
        return self.x(self.slot_x[slot])

    def W(self, slot: int) -> torch.Tensor:
        """Out-major base weight of ``slot``: element (k, n) of W is ``W(slot)[n, k]``."""
        key = ("W", slot)
        if key not in self._cache:
            self._cache[key] = _draw((self.hidden, self.hidden), self.w_std,
                                     _seed(self.master, _K_W, slot), self.dtype, self.device, self.values)
        return self._cache[key]

    def _draw_ab(self, aid: int):
        r = int(self.ranks[aid])
        shape = (self.n_slots, r, self.hidden)
        return (_draw(shape, self.ab_std, _seed(self.master, _K_AB, aid, 0), self.dtype, self.device, self.values),
                _draw(shape, self.ab_std, _seed(self.master, _K_AB, aid, 1), self.dtype, self.device, self.values))

    def adapter(self, aid: int):
        """(A_t, B), each [n_slots][r][H]; r = ranks[aid] (may be 0)."""
        key = ("AB", aid)
        if key not in self._cache:
            self._cache[key] = self._draw_ab(aid)
        return self._cache[key]

    def adapter_uncached(self, aid: int):
        """The same (A_t, B) as ``adapter`` (same seeds, same values), drawn without keeping them: for
        loading pools whose adapters would not fit twice in memory."""
        return self._cache.get(("AB", aid)) or self._draw_ab(aid)

    def drop_cache(self, kind: str | None = None) -> None:
        for k in list(self._cache):
            if kind is None or k[0] == kind:
                del self._cache[k]

    def kv_canary(self, n: int) -> torch.Tensor:
        """Seeded bit pattern written into KV pages to check they are never modified."""
        g = torch.Generator(device=self.device).manual_seed(_seed(self.master, _K_CANARY))
        return torch.randint(-2**15, 2**15, (n, self.hidden * self.elem // 2), generator=g,
                             device=self.device, dtype=torch.int32).to(torch.int16)


# ---------------------------------------------------------------------------------------
# pool plans
#
# ops (executed in order against a pool created with ``free_order``):
#   ("load", aid)            load adapter aid at rank ranks[aid] over all slots
#   ("kv", rid, layers)      grow request rid's KV by one token (2*layers pages)
#   ("free_kv", rid)         request rid finished: its KV pages return to the free list
#   ("release", aid)         one request of adapter aid finished (refcount - 1)
#   ("evict", aid)           return an idle adapter's pages to the free list
# ---------------------------------------------------------------------------------------

def _interleaved_plan(rng, adapters, ranks, n_slots, kv_share, adapter_share, kv_layers):
    adapter_pages = int(sum(2 * int(ranks[a]) * n_slots for a in adapters))
    num_pages = max(1, math.ceil(adapter_pages / adapter_share))
    kv_grow = 2 * kv_layers
    n_kv = min(round(kv_share * num_pages / kv_grow), (num_pages - adapter_pages) // kv_grow)
    ops = [("load", int(a)) for a in adapters] + [("kv", i, kv_layers) for i in range(n_kv)]
    order = rng.permutation(len(ops))
    ops = [ops[i] for i in order]
    free_order = rng.permutation(num_pages).astype(np.int64)
    return num_pages, free_order, ops


def _churn_plan(rng, adapters, ranks, n_slots, kv_layers, rounds=4):
    """Seeded alloc/free churn: KV requests of varying length and adapter loads/evictions."""
    adapter_pages = int(sum(2 * int(ranks[a]) * n_slots for a in adapters))
    num_pages = math.ceil(adapter_pages / 0.80)
    kv_cap = int(0.15 * num_pages)
    kv_grow = 2 * kv_layers
    free_order = rng.permutation(num_pages).astype(np.int64)
    ops = []
    kv_live = {}          # rid -> pages
    loaded = []
    next_rid = 0

    def top_up_kv():
        nonlocal next_rid
        while True:
            toks = int(rng.integers(1, 51))
            pages = toks * kv_grow
            if sum(kv_live.values()) + pages > kv_cap:
                return
            ops.extend(("kv", next_rid, kv_layers) for _ in range(toks))
            kv_live[next_rid] = pages
            next_rid += 1

    for _ in range(rounds):
        top_up_kv()
        not_loaded = [a for a in adapters if a not in loaded]
        pick = rng.permutation(len(not_loaded))[: len(not_loaded) // 2]
        for i in sorted(pick):
            ops.append(("load", int(not_loaded[i])))
            loaded.append(int(not_loaded[i]))
        rids = sorted(kv_live)
        for i in rng.permutation(len(rids))[: len(rids) // 2]:
            ops.append(("free_kv", rids[i]))
            del kv_live[rids[i]]
        for i in sorted(rng.permutation(len(loaded))[: len(loaded) // 2], reverse=True):
            a = loaded.pop(i)
            ops.append(("release", a))
            ops.append(("evict", a))
    for a in adapters:
        if a not in loaded:
            ops.append(("load", int(a)))
            loaded.append(int(a))
    top_up_kv()
    return num_pages, free_order, ops


# ---------------------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------------------

def build(name: str, device: str = "cpu", layers: int | None = None) -> Workload:
    """One of the five named workloads.  ``layers`` (stack13b only) keeps the first ``layers``
    of the 40 layers (4 q/k/v/o slots each); everything else -- ids, ranks, pool plan rules --
    is the same."""
    m = _MASTER[name]
    if layers is not None and name != "stack13b":
        raise ValueError("layers applies to stack13b only")
    r_ids, r_ranks, r_pool = _rng(m, _K_IDS), _rng(m, _K_RANKS), _rng(m, _K_POOL)
    if name == "tiny":
        H, dt, n_slots, n_ad, T = 256, "f32", 1, 4, 16
        ranks = np.array([4, 8, 8, 16], np.int32)
        ids = r_ids.integers(0, n_ad, T).astype(np.int32)
        slot_x, n_x, segs = [0], 1, []
        adapters = list(range(n_ad))
        plan = _interleaved_plan(r_pool, adapters, ranks, n_slots, 0.60, 0.35, kv_layers=1)
    elif name == "decode":
        H, dt, n_slots, n_ad, T = 4096, "bf16", 1, 32, 64
        ranks = r_ranks.choice(np.array([8, 16, 32, 64], np.int32), n_ad).astype(np.int32)
        ids = r_ids.integers(0, n_ad, T).astype(np.int32)
        slot_x, n_x, segs = [0], 1, []
        adapters = list(range(n_ad))
        plan = _interleaved_plan(r_pool, adapters, ranks, n_slots, 0.60, 0.35, kv_layers=32)
    elif name == "prefill":
        H, dt, n_slots, n_ad, T = 4096, "bf16", 1, 8, 4096
        ranks = np.array([8, 8, 16, 16, 32, 32, 64, 64], np.int32)
        ids = np.repeat(np.arange(n_ad, dtype=np.int32), 512)
        slot_x, n_x = [0], 1
        segs = [(512 * i, 512) for i in range(n_ad)]
        adapters = list(range(n_ad))
        plan = _interleaved_plan(r_pool, adapters, ranks, n_slots, 0.60, 0.35, kv_layers=32)
    elif name == "many":
        H, dt, n_slots, T = 4096, "bf16", 4, 256
        n_real = 2000
        n_ad = n_real + 1                      # id 2000 is the identity (rank-0) adapter
        ranks = np.concatenate([r_ranks.choice(np.array([8, 16, 32, 64], np.int32), n_real),
                                np.zeros(1, np.int32)]).astype(np.int32)
        n_ident = round(0.1 * T)
        ids = _finite_zipf(r_ids, n_real, 1.0, T)
        ids[r_ids.permutation(T)[:n_ident]] = n_real
        slot_x, n_x, segs = [0, 0, 0, 1], 2, []
        adapters = list(range(n_ad))
        plan = _interleaved_plan(r_pool, adapters, ranks, n_slots, 0.60, 0.35, kv_layers=32)
    elif name == "stack13b":
        H, dt = 5120, "bf16"
        n_slots = 4 * (40 if layers is None else int(layers))
        if not 1 <= n_slots // 4 <= 40:
            raise ValueError("layers must be in 1..40")
        n_ad = 1000
        ranks = r_ranks.choice(np.array([8, 16, 32, 64], np.int32), n_ad).astype(np.int32)
        pre = _finite_zipf(r_ids, n_ad, 1.2, 4)
        dec = _finite_zipf(r_ids, n_ad, 1.2, 256)
        ids = np.concatenate([np.repeat(pre, 2048), dec]).astype(np.int32)
        T = int(ids.size)
        slot_x, n_x = [0 if s % 4 != 3 else 1 for s in range(n_slots)], 2
        segs = [(2048 * i, 2048) for i in range(4)]
        adapters = list(range(n_ad))
        plan = _churn_plan(r_pool, adapters, ranks, n_slots, kv_layers=40)
    else:
        raise KeyError(name)
    scales = np.where(ranks > 0, 16.0 / np.maximum(ranks, 1), 0.0).astype(np.float32)
    num_pages, free_order, ops = plan
    return Workload(name=name, hidden=H, dtype=dt, n_slots=n_slots, max_adapters=n_ad, T=T,
                    ids=ids, ranks=ranks, scales=scales, slot_x=slot_x, n_x=n_x,
                    num_pages=num_pages, free_order=free_order, ops=ops, master=m,
                    device=device, segments=segs)


def custom(hidden: int, ranks, ids, *, dtype: str = "bf16", n_slots: int = 1, seed: int = 7,
           values: str = "normal", scales=None, kv_share: float = 0.60, kv_layers: int = 1,
           slot_x=None, n_x: int = 1, device: str = "cpu", w_std: float = 0.02,
           ab_std: float = 0.02, x_std: float = 1.0, load=None) -> Workload:
    """A small workload for tests.  ``ranks[a]`` per adapter; ``ids`` per token (-1 = none).

    ``load`` lists the adapters to place in the pool (default: all); ``scales`` defaults to 16/r.
    """
    ranks = np.asarray(ranks, np.int32)
    ids = np.asarray(ids, np.int32)
    n_ad = int(ranks.size)
    if scales is None:
        scales = np.where(ranks > 0, 16.0 / np.maximum(ranks, 1), 0.0)
    scales = np.asarray(scales, np.float32)
    adapters = list(range(n_ad)) if load is None else list(load)
    r_pool = _rng(seed, _K_POOL)
    num_pages, free_order, ops = _interleaved_plan(r_pool, adapters, ranks, n_slots, kv_share,
                                                   0.35, kv_layers)
    if num_pages < 1:
        num_pages = 1
    return Workload(name=f"custom{seed}", hidden=hidden, dtype=dtype, n_slots=n_slots,
                    max_adapters=n_ad, T=int(ids.size), ids=ids, ranks=ranks, scales=scales,
                    slot_x=list(slot_x) if slot_x is not None else [0] * n_slots, n_x=n_x,
                    num_pages=num_pages, free_order=free_order, ops=ops, master=seed,
                    device=device, values=values, w_std=w_std, ab_std=ab_std, x_std=x_std)
