"""A model of the unified page pool, and the memory arithmetic around it.  Test infrastructure only.

Source: "S-LoRA, in depth", section "Unified paging: adapters and KV cache in one pool", its
worked example and its pool sketch.  Behaviour restated here:
  * the pool starts with every page on one free list; allocations take pages from the end of the
    list, frees append to it (the sketch's list pop / extend);
  * an adapter of rank r on P projections of L layers takes r*2*P*L pages (A and B per projection);
  * admitting a request for a resident adapter only counts one more user; a new adapter first
    evicts idle adapters (no users, oldest first) when pages are short, and fails when even that
    is not enough -- the idle adapters evicted on the way stay evicted;
  * one more KV token takes 2*L pages (K and V per layer) and fails when pages are short;
  * a finished request returns its KV pages; an idle adapter's pages can be reclaimed.

Extensions beyond the sketch (each an explicit reading):
  * the initial free list may be any permutation of the page ids (seeded random placement);
  * ``n_slots`` = layers * projections; within one adapter's page list, slot s owns entries
    [2 r s, 2 r (s+1)), A's columns first then B's rows;
  * reloading a resident adapter at a different rank is an error ("eexist");
  * ``release`` drops one user, ``evict`` reclaims one idle adapter, ``free_kv`` ends a request;
  * the order in which idle adapters are evicted (the victim rule) is selectable:
      - "load_order": oldest load first, the sketch's rule (an adapter evicted and loaded again
        counts from its new load);
      - "lru": least recently used first, where a use is an admission (``ensure_adapter``) --
        the rule the MoE-offload page ("Cache the Experts You Will Need") measures as LRU;
      - "farthest": the adapter whose next request in the caller's lookahead (upcoming adapter
        ids, soonest first) lies farthest, as Belady's rule on that page; adapters with no request
        in the lookahead count as farthest and, as in its "Limited foresight" paragraph, are
        ordered among themselves least recently used first; ties inside the lookahead cannot occur
        (each position names one adapter).
"""
from __future__ import annotations

import numpy as np


# ---- memory arithmetic (section "Unified paging", worked example) -------------------------

def pages_for_adapter(rank: int, layers: int, projections: int) -> int:
    """A and B per projection, each r vectors of length H."""
    return rank * 2 * projections * layers


def kv_pages_per_token(layers: int) -> int:
    """K and V: one vector each per layer."""
    return 2 * layers


def kv_bytes_per_token(layers: int, hidden: int, elem_bytes: int) -> int:
    return kv_pages_per_token(layers) * hidden * elem_bytes


def adapter_bytes(rank: int, layers: int, projections: int, hidden: int, elem_bytes: int) -> int:
    return pages_for_adapter(rank, layers, projections) * hidden * elem_bytes


def h2d_seconds(nbytes: float, bytes_per_second: float) -> float:
    """Copy time of an adapter over a link of the given rate (section "Scheduling", prefetching)."""
    return nbytes / bytes_per_second


def tp_comm_lora(n_gpus: int, tokens: int, rank: int) -> float:
    """Added traffic of the adapter layout under tensor parallelism (section "Tensor parallelism
    for adapters"): three all-gathers and one all-reduce of width r."""
    return 5 * (n_gpus - 1) * tokens * rank / n_gpus


def tp_comm_base(n_gpus: int, tokens: int, hidden: int) -> float:
    return 2 * (n_gpus - 1) * tokens * hidden / n_gpus


# ---- the pool ------------------------------------------------------------------------------

class UnifiedPoolModel:
    """Host-side page bookkeeping of one pool; page contents are not modelled."""

    VICTIM_RULES = ("load_order", "lru", "farthest")

    def __init__(self, num_pages: int, free_order=None, victim: str = "load_order"):
        assert victim in self.VICTIM_RULES, victim
        self.victim = victim
        self.lookahead: list[int] = []
        self.tick = 0
        self.last_use: dict[int, int] = {}
        self.num_pages = int(num_pages)
        if free_order is None:
            self.free = list(range(self.num_pages))
        else:
            self.free = [int(p) for p in free_order]
            assert sorted(self.free) == list(range(self.num_pages)), "free_order must be a permutation"
        self.adapter_pages: dict[int, list[int]] = {}   # insertion order = load order
        self.adapter_rank: dict[int, int] = {}
        self.adapter_refs: dict[int, int] = {}
        self.kv_pages: dict[int, list[int]] = {}

    def _take(self, n: int) -> list:
        return [self.free.pop() for _ in range(n)]

    def set_lookahead(self, ids) -> None:
        """Upcoming adapter requests, soonest first (the waiting queue a scheduler can see)."""
        self.lookahead = [int(a) for a in ids]

    def ensure_adapter(self, aid: int, rank: int, n_slots: int) -> str:
        if aid in self.adapter_pages:
            if self.adapter_rank[aid] != rank:
                return "eexist"
            self.adapter_refs[aid] += 1
            self.tick += 1
            self.last_use[aid] = self.tick
            return "ok"
        need = 2 * rank * n_slots
        if len(self.free) < need and not self.evict_idle_adapters(need):
            return "enomem"
        self.adapter_pages[aid] = self._take(need)
        self.adapter_rank[aid] = rank
        self.adapter_refs[aid] = 1
        self.tick += 1
        self.last_use[aid] = self.tick
        return "ok"

    def victim_order(self) -> list:
        """The idle adapters in the order the victim rule evicts them."""
        idle = [a for a, n in self.adapter_refs.items() if n == 0]   # load order
        if self.victim == "lru":
            idle.sort(key=lambda a: self.last_use[a])
        elif self.victim == "farthest":
            far = len(self.lookahead)
            def next_use(a):
                return self.lookahead.index(a) if a in self.lookahead else far
            idle.sort(key=lambda a: (-next_use(a), self.last_use[a]))
        return idle

    def evict_idle_adapters(self, need: int) -> bool:
        for aid in self.victim_order():
            self._drop(aid)
            if len(self.free) >= need:
                return True
        return len(self.free) >= need

    def _drop(self, aid: int) -> None:
        self.free.extend(self.adapter_pages.pop(aid))
        del self.adapter_refs[aid]
        del self.adapter_rank[aid]
        del self.last_use[aid]

    def release(self, aid: int) -> str:
        if aid not in self.adapter_refs:
            return "enoent"
        if self.adapter_refs[aid] == 0:
            return "einval"
        self.adapter_refs[aid] -= 1
        return "ok"

    def evict(self, aid: int) -> str:
        if aid not in self.adapter_refs:
            return "enoent"
        if self.adapter_refs[aid] > 0:
            return "ebusy"
        self._drop(aid)
        return "ok"

    def grow_kv(self, rid: int, layers: int) -> str:
        need = kv_pages_per_token(layers)
        if len(self.free) < need:
            return "enomem"
        self.kv_pages.setdefault(rid, []).extend(self._take(need))
        return "ok"

    def free_kv(self, rid: int) -> str:
        if rid not in self.kv_pages:
            return "enoent"
        self.free.extend(self.kv_pages.pop(rid))
        return "ok"

    # ---- views ---------------------------------------------------------------------------
    def run(self, ops, ranks, n_slots: int) -> list:
        """Apply a workload's operation list; returns each operation's status."""
        out = []
        for op in ops:
            kind = op[0]
            if kind == "load":
                out.append(self.ensure_adapter(op[1], int(ranks[op[1]]), n_slots))
            elif kind == "kv":
                out.append(self.grow_kv(op[1], op[2]))
            elif kind == "free_kv":
                out.append(self.free_kv(op[1]))
            elif kind == "release":
                out.append(self.release(op[1]))
            elif kind == "evict":
                out.append(self.evict(op[1]))
            else:
                raise ValueError(kind)
        return out

    def page_table(self, slot: int, max_adapters: int, max_rank: int) -> np.ndarray:
        """[max_adapters][2*max_rank]: slot's A-column pages then B-row pages, -1 padded."""
        pt = np.full((max_adapters, 2 * max_rank), -1, dtype=np.int64)
        for aid, pages in self.adapter_pages.items():
            r = self.adapter_rank[aid]
            pt[aid, : 2 * r] = pages[2 * r * slot: 2 * r * (slot + 1)]
        return pt

    def kv_page_set(self) -> set:
        return {p for pages in self.kv_pages.values() for p in pages}

    def stats(self) -> dict:
        return {
            "num_pages": self.num_pages,
            "free_pages": len(self.free),
            "kv_pages": sum(len(v) for v in self.kv_pages.values()),
            "adapter_pages": sum(len(v) for v in self.adapter_pages.values()),
            "resident_adapters": len(self.adapter_pages),
        }
