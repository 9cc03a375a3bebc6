"""Pins of the pool model and the memory arithmetic: the worked example's printed values, a trace
derived by hand from the pool sketch, and invariants under random operation sequences."""
import json
import os

import numpy as np
import pytest

from oracle import (PagePoolModel, adapter_bytes, gather_page_ids, expected_page_rows,
                    h2d_seconds, kv_bytes_per_token, kv_pages_per_token, adapter_page_count,
                    tp_comm_base, tp_comm_lora)

KiB, MiB, GiB = 1024, 1024 ** 2, 1024 ** 3


@pytest.fixture
def worked(golden_dir):
    with open(os.path.join(golden_dir, "slora_worked_example.json")) as f:
        return json.load(f)


@pytest.fixture
def traces(golden_dir):
    with open(os.path.join(golden_dir, "pool_trace.json")) as f:
        return json.load(f)["traces"]


def test_worked_example_kv(worked):
    m = worked["model"]
    assert kv_pages_per_token(m["layers"]) == worked["kv_vectors_per_token"]
    assert kv_bytes_per_token(m["layers"], m["hidden"], m["elem_bytes"]) == worked["kv_bytes_per_token"]
    assert worked["kv_bytes_per_token"] == 512 * KiB


def test_worked_example_adapter(worked):
    m, a = worked["model"], worked["adapter"]
    assert adapter_page_count(a["rank"], 1, a["projections"]) == worked["adapter_vectors_per_layer"]
    assert adapter_page_count(a["rank"], m["layers"], a["projections"]) == worked["adapter_vectors_total"]
    nbytes = adapter_bytes(a["rank"], m["layers"], a["projections"], m["hidden"], m["elem_bytes"])
    assert nbytes == worked["adapter_bytes"] == 32 * MiB
    kv = kv_bytes_per_token(m["layers"], m["hidden"], m["elem_bytes"])
    assert nbytes // kv == worked["kv_tokens_per_adapter"] and nbytes % kv == 0


def test_worked_example_rounded_figures(worked):
    m, a = worked["model"], worked["adapter"]
    nbytes = adapter_bytes(a["rank"], m["layers"], a["projections"], m["hidden"], m["elem_bytes"])
    kv = kv_bytes_per_token(m["layers"], m["hidden"], m["elem_bytes"])
    per_ctx = worked["context_tokens"] * kv / nbytes           # 31.25: "about 31"
    assert round(per_ctx) == worked["adapters_per_context_approx"]
    total_gib = worked["n_adapters"] * nbytes / GiB              # 62.5: "about 62"
    assert int(total_gib) == worked["all_adapters_gib_approx"]
    p = worked["prefetch"]
    ms = 1e3 * h2d_seconds(p["adapter_bytes"], p["link_bytes_per_s"])   # 1.68: "roughly 1.6 ms"
    assert abs(ms - p["copy_ms_approx"]) < 0.1


def test_tensor_parallel_ratio(worked):
    tp = worked["tensor_parallel"]
    for n in (2, 4, 8):
        ratio = tp_comm_lora(n, 64, tp["rank"]) / tp_comm_base(n, 64, tp["hidden"])
        assert ratio == pytest.approx(5 * 16 / (2 * 4096)) and ratio < tp["ratio_bound"]


def test_rank_slot_ratio(worked):
    r = worked["rank_slot_ratio"]
    assert adapter_page_count(r["big_rank"], 32, 4) == r["ratio"] * adapter_page_count(r["small_rank"], 32, 4)


def _apply(pool, step, n_slots):
    op = step["op"]
    if op == "load":
        before = list(pool.free_list)
        st = pool.admit(step["aid"], step["rank"], n_slots)
        res = pool.residents.get(step["aid"])
        taken = [] if st != "ok" or res.users > 1 else res.pages
        return st, taken, before
    if op == "kv":
        n0 = len(pool.requests.get(step["rid"], []))
        st = pool.add_kv_token(step["rid"], step["layers"])
        return st, pool.requests.get(step["rid"], [])[n0:], None
    if op == "free_kv":
        return pool.end_request(step["rid"]), None, None
    if op == "release":
        return pool.release(step["aid"]), None, None
    if op == "evict":
        return pool.evict(step["aid"]), None, None
    raise ValueError(op)


def test_hand_derived_traces(traces):
    for tr in traces:
        pool = PagePoolModel(tr["num_pages"])
        for step in tr["steps"]:
            st, taken, _ = _apply(pool, step, tr["n_slots"])
            assert st == step["status"], step
            if "pages" in step:
                assert list(taken or []) == step["pages"], step
        fin = tr["final"]
        assert pool.free_list == fin["free"]
        assert pool.resident_ids() == fin["resident_in_load_order"]
        assert {str(k): v for k, v in pool.requests.items()} == fin["kv"]
        for key in [k for k in fin if k.startswith("page_table_slot")]:
            slot = int(key[len("page_table_slot"):])
            pt = pool.page_table(slot, tr["max_adapters"], tr["max_rank"])
            for a, row in fin[key].items():
                assert list(pt[int(a)]) == row, (key, a)


def test_random_ops_invariants():
    rng = np.random.default_rng(0)
    for trial in range(20):
        n = int(rng.integers(10, 200))
        pool = PagePoolModel(n, rng.permutation(n))
        n_slots = int(rng.integers(1, 4))
        for _ in range(200):
            k = rng.integers(0, 5)
            if k == 0:
                pool.admit(int(rng.integers(0, 8)), int(rng.integers(0, 5)), n_slots)
            elif k == 1:
                pool.add_kv_token(int(rng.integers(0, 6)), int(rng.integers(1, 3)))
            elif k == 2:
                pool.end_request(int(rng.integers(0, 6)))
            elif k == 3:
                pool.release(int(rng.integers(0, 8)))
            else:
                pool.evict(int(rng.integers(0, 8)))
            used = [p for r in pool.residents.values() for p in r.pages] + [p for v in pool.requests.values() for p in v]
            every = used + pool.free_list
            assert sorted(every) == list(range(n))          # conserved and pairwise distinct
            for aid, res in pool.residents.items():
                assert len(res.pages) == 2 * res.rank * n_slots
                assert res.users >= 0


def test_gather_ids_hand_table():
    pt = np.array([[5, 9, 2, 7], [-1, -1, -1, -1], [3, 4, -1, -1]])
    ranks = np.array([2, 0, 1])
    got = gather_page_ids(pt, np.array([2, -1, 0, 1, 0]), ranks, max_rank=2)
    want = np.array([[3, 4, -1, -1], [-1] * 4, [5, 9, 2, 7], [-1] * 4, [5, 9, 2, 7]])
    assert np.array_equal(got, want)


def test_expected_page_rows():
    pt = np.array([[5, 9, 2, 7]])
    At = np.arange(8).reshape(2, 4)
    B = 100 + np.arange(8).reshape(2, 4)
    rows = expected_page_rows(pt, 0, 2, At, B)
    assert [p for p, _ in rows] == [5, 9, 2, 7]
    assert np.array_equal(rows[0][1], At[0]) and np.array_equal(rows[3][1], B[1])


# ---- victim rules ------------------------------------------------------------------------------
# Three adapters of rank 2 on one slot (4 pages each) fill a 12-page pool.  Worked by hand from
# the rules' definitions (oracle/pool.py header): after "0, 1, 2 loaded and released, then 0
# admitted again and released", a fourth adapter needs 4 pages and one idle adapter must go.
#   load order: 0 was loaded first (its second admission is not a load)            -> evict 0
#   lru:        last uses 0 @4, 1 @2, 2 @3                                          -> evict 1
#   farthest, lookahead [1, 0, 2]: next uses 1 @0, 0 @1, 2 @2                       -> evict 2
#   farthest, lookahead [1]: 0 and 2 are beyond it, least recently used of them     -> evict 2
#   farthest, lookahead [2]: 0 and 1 are beyond it, least recently used of them     -> evict 1
@pytest.mark.parametrize("victim,lookahead,evicted", [
    ("load_order", [], 0), ("lru", [], 1), ("farthest", [1, 0, 2], 2), ("farthest", [1], 2),
    ("farthest", [2], 1), ("farthest", [], 1)])
def test_victim_rules_hand_trace(victim, lookahead, evicted):
    m = PagePoolModel(12, victim=victim)
    for a in (0, 1, 2, 0):
        assert m.admit(a, 2, 1) == "ok"
        assert m.release(a) == "ok"
    m.set_lookahead(lookahead)
    assert m.admit(3, 2, 1) == "ok"
    assert sorted(m.resident_ids()) == sorted({0, 1, 2, 3} - {evicted})
    assert len(m.free_list) == 0


def _min_loads(seq, cap):
    """Fewest loads any schedule needs to serve `seq` one request at a time with room for `cap`
    adapters: exhaustive search over every choice of victim (memoised on the resident set)."""
    from functools import lru_cache

    @lru_cache(maxsize=None)
    def f(i, res):
        if i == len(seq):
            return 0
        a = seq[i]
        if a in res:
            return f(i + 1, res)
        if len(res) < cap:
            return 1 + f(i + 1, res | {a})
        return 1 + min(f(i + 1, (res - {v}) | {a}) for v in res)
    return f(0, frozenset())


def _loads(seq, cap, victim, foresight=None):
    """Loads the pool model makes serving `seq` (admit, then release, each request), adapters of
    rank 1 on one slot (2 pages each), `cap` of them fitting."""
    m = PagePoolModel(2 * cap, victim=victim)
    n = 0
    for i, a in enumerate(seq):
        rest = seq[i + 1:]
        m.set_lookahead(rest if foresight is None else rest[:foresight])
        n += a not in m.residents
        assert m.admit(a, 1, 1) == "ok"
        assert m.release(a) == "ok"
    return n


def test_farthest_with_full_lookahead_is_optimal():
    """For one request at a time and equal sizes, evicting the adapter needed farthest in the future
    makes the fewest loads (Belady's rule, cited on the MoE-offload page); checked against the
    exhaustive search on random short traces, and no other rule does better."""
    rng = np.random.default_rng(7)
    worse = 0
    for trial in range(120):
        cap = int(rng.integers(2, 4))
        seq = [int(a) for a in rng.integers(0, cap + 3, int(rng.integers(6, 13)))]
        best = _min_loads(tuple(seq), cap)
        assert _loads(seq, cap, "farthest") == best, (seq, cap)
        for victim in ("lru", "load_order"):
            got = _loads(seq, cap, victim)
            assert got >= best
            worse += got > best
        assert _loads(seq, cap, "farthest", foresight=1) >= best
    assert worse > 0   # the traces do separate the rules
