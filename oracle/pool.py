"""A model of the unified page pool, and the memory arithmetic around it.  Test infrastructure only.

Source: "S-LoRA, in depth", section "Unified paging: adapters and KV cache in one pool", its worked
example and its pool sketch.  What the pool must do, restated:
  * all pages start on one free list; pages are handed out from the end of the list and handed
    back by appending to it, in the order of the list they came from;
  * an adapter of rank r on P projections of L layers takes r*2*P*L pages (A and B per projection);
  * admitting a request whose adapter is already resident only adds a user; a new adapter, when
    pages are short, first reclaims idle adapters (no users) one by one until enough are free, and
    is refused when even that is not enough (what was reclaimed on the way stays reclaimed);
  * one more KV token of a request takes 2*L pages (K and V per layer), and is refused when pages
    are short;
  * a finished request hands back its KV pages; an idle adapter's pages can be reclaimed.

Extensions beyond the page (each an explicit reading):
  * the initial free list may be any permutation of the page ids (seeded random placement);
  * ``n_slots`` = layers * projections; within one adapter's page list, slot s owns entries
    [2 r s, 2 r (s+1)), A's columns first then B's rows;
  * admitting a resident adapter at a different rank is an error ("eexist");
  * ``release`` drops one user, ``evict`` reclaims one idle adapter, ``end_request`` returns a
    request's KV pages;
  * the order in which idle adapters are reclaimed (the victim rule) is selectable:
      - "load_order": oldest load first, the page's rule (an adapter reclaimed and loaded again
        counts from its new load);
      - "lru": least recently admitted first -- the rule the MoE-offload page ("Cache the Experts
        You Will Need") measures as LRU;
      - "farthest": the adapter whose next request in the caller's lookahead (upcoming adapter ids,
        soonest first) lies farthest, Belady's rule on that page; adapters the lookahead does not
        name count as farthest and, as in its "Limited foresight" paragraph, go least recently
        admitted first among themselves.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


# ---- memory arithmetic (section "Unified paging", worked example) -------------------------

def adapter_page_count(rank: int, layers: int, projections: int) -> int:
    """Pages of one adapter: A and B on every projection of every layer, r vectors of length H each."""
    return layers * projections * (2 * rank)


def kv_pages_per_token(layers: int) -> int:
    """K and V: one vector each per layer."""
    return 2 * layers


def kv_bytes_per_token(layers: int, hidden: int, elem_bytes: int) -> int:
    return kv_pages_per_token(layers) * hidden * elem_bytes


def adapter_bytes(rank: int, layers: int, projections: int, hidden: int, elem_bytes: int) -> int:
    return adapter_page_count(rank, layers, projections) * hidden * elem_bytes


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

@dataclass
class Resident:
    """One adapter holding pages: its rank, its users, its page list and when it was last admitted."""
    rank: int
    pages: list
    users: int = 1
    admitted: int = 0


@dataclass
class PagePoolModel:
    """Host-side page bookkeeping of one pool; page contents are not modelled.

    ``residents`` keeps adapters in load order (dict insertion order); ``requests`` maps a request
    id to its KV pages in the order they were handed out."""

    num_pages: int
    free_order: object = None
    victim: str = "load_order"
    free_list: list = field(init=False)
    residents: dict = field(init=False, default_factory=dict)
    requests: dict = field(init=False, default_factory=dict)
    lookahead: list = field(init=False, default_factory=list)
    clock: int = field(init=False, default=0)

    VICTIM_RULES = ("load_order", "lru", "farthest")

    def __post_init__(self):
        assert self.victim in self.VICTIM_RULES, self.victim
        self.num_pages = int(self.num_pages)
        if self.free_order is None:
            self.free_list = list(range(self.num_pages))
        else:
            self.free_list = [int(p) for p in self.free_order]
            assert sorted(self.free_list) == list(range(self.num_pages)), "free_order must be a permutation"

    # ---- page movement ------------------------------------------------------------------
    def _hand_out(self, n: int) -> list:
        """The last n free pages, the very last one first."""
        cut = len(self.free_list) - n
        taken = self.free_list[cut:][::-1]
        del self.free_list[cut:]
        return taken

    def _hand_back(self, pages) -> None:
        self.free_list += list(pages)

    def _reclaim(self, aid: int) -> None:
        self._hand_back(self.residents.pop(aid).pages)

    def _make_room(self, need: int) -> bool:
        """Reclaim idle adapters, in victim order, while fewer than `need` pages are free."""
        victims = iter(self.eviction_order())
        while len(self.free_list) < need:
            aid = next(victims, None)
            if aid is None:
                return False
            self._reclaim(aid)
        return True

    # ---- operations ---------------------------------------------------------------------
    def set_lookahead(self, ids) -> None:
        """Upcoming adapter requests, soonest first (the waiting queue a scheduler can see)."""
        self.lookahead = [int(a) for a in ids]

    def eviction_order(self) -> list:
        """The idle adapters in the order the victim rule reclaims them."""
        idle = [aid for aid, res in self.residents.items() if res.users == 0]   # load order
        if self.victim == "lru":
            idle.sort(key=lambda aid: self.residents[aid].admitted)
        elif self.victim == "farthest":
            soonest = {}
            for pos, aid in enumerate(self.lookahead):
                soonest.setdefault(aid, pos)
            beyond = len(self.lookahead)
            idle.sort(key=lambda aid: (-soonest.get(aid, beyond), self.residents[aid].admitted))
        return idle

    def admit(self, aid: int, rank: int, n_slots: int) -> str:
        """A request for adapter `aid` at `rank` arrives: one more user, loading it if needed."""
        self.clock += 1
        res = self.residents.get(aid)
        if res is not None:
            if res.rank != rank:
                return "eexist"
            res.users += 1
            res.admitted = self.clock
            return "ok"
        need = 2 * rank * n_slots
        if not self._make_room(need):
            return "enomem"
        self.residents[aid] = Resident(rank=rank, pages=self._hand_out(need), admitted=self.clock)
        return "ok"

    def add_kv_token(self, rid: int, layers: int) -> str:
        need = kv_pages_per_token(layers)
        if len(self.free_list) < need:
            return "enomem"
        self.requests[rid] = self.requests.get(rid, []) + self._hand_out(need)
        return "ok"

    def end_request(self, rid: int) -> str:
        if rid not in self.requests:
            return "enoent"
        self._hand_back(self.requests.pop(rid))
        return "ok"

    def release(self, aid: int) -> str:
        res = self.residents.get(aid)
        if res is None:
            return "enoent"
        if res.users == 0:
            return "einval"
        res.users -= 1
        return "ok"

    def evict(self, aid: int) -> str:
        res = self.residents.get(aid)
        if res is None:
            return "enoent"
        if res.users > 0:
            return "ebusy"
        self._reclaim(aid)
        return "ok"

    def run(self, ops, ranks, n_slots: int) -> list:
        """Apply a workload's operation list; returns each operation's status."""
        handlers = {
            "load": lambda op: self.admit(op[1], int(ranks[op[1]]), n_slots),
            "kv": lambda op: self.add_kv_token(op[1], op[2]),
            "free_kv": lambda op: self.end_request(op[1]),
            "release": lambda op: self.release(op[1]),
            "evict": lambda op: self.evict(op[1]),
        }
        return [handlers[op[0]](op) for op in ops]

    # ---- views ---------------------------------------------------------------------------
    def resident_ids(self) -> list:
        """Resident adapters in load order."""
        return list(self.residents)

    def pages_of(self, aid: int) -> list:
        return self.residents[aid].pages

    def page_table(self, slot: int, max_adapters: int, max_rank: int) -> np.ndarray:
        """[max_adapters][2*max_rank]: slot's A-column pages then B-row pages, -1 padded."""
        pt = np.full((max_adapters, 2 * max_rank), -1, dtype=np.int64)
        for aid, res in self.residents.items():
            width = 2 * res.rank
            pt[aid, :width] = res.pages[width * slot: width * (slot + 1)]
        return pt

    def kv_page_set(self) -> set:
        return {p for pages in self.requests.values() for p in pages}

    def stats(self) -> dict:
        return {
            "num_pages": self.num_pages,
            "free_pages": len(self.free_list),
            "kv_pages": sum(len(v) for v in self.requests.values()),
            "adapter_pages": sum(len(r.pages) for r in self.residents.values()),
            "resident_adapters": len(self.residents),
        }
