"""The C-ABI library on the CPU: it loads, exports every declared symbol, and its host-side pool
bookkeeping matches the oracle's pool model bit for bit.  No device work is done here (pools are
bookkeeping-only: no pages, no page table)."""
import ctypes
import json
import os
import re
import subprocess

import numpy as np
import pytest

import rank_gemm_unified_amd as rg
from oracle import PagePoolModel, kv_pages_per_token, adapter_page_count
from workloads import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lorapool.h")

_STATUS = {"ok": 0, "enomem": -2, "enoent": -3, "ebusy": -5, "eexist": -6, "einval": -1}


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(lora_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 20, names
    out = subprocess.run(["nm", "-D", "--defined-only", rg.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s+(lora_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(rg.EXPORTED) == set(names)


def test_version_and_constants():
    assert "gfx950" in rg.lora_version()
    assert rg.SOURCE_HASH and rg.lora_version().endswith(" src " + rg.SOURCE_HASH)
    text = open(HEADER).read()
    assert f"#define LORA_MAX_RANK {rg.LORA_MAX_RANK}" in text
    assert re.search(rf"#define LORA_MAX_ADAPTERS {rg.LORA_MAX_ADAPTERS}\b", text)
    assert "#define LORA_MAX_TOKENS (1 << 22)" in text and rg.LORA_MAX_TOKENS == 1 << 22


def test_library_built_from_other_sources_is_refused(tmp_path):
    """A copy of the package whose sources no longer match its library: importing it fails."""
    import shutil
    import sys
    pkg = os.path.dirname(os.path.abspath(rg.__file__))
    shutil.copytree(pkg, tmp_path / "rank_gemm_unified_amd", ignore=shutil.ignore_patterns("_build", "__pycache__"))
    (tmp_path / "include").mkdir()
    shutil.copy(HEADER, tmp_path / "include" / "lorapool.h")
    probe = "import rank_gemm_unified_amd as r; print(r.SOURCE_HASH)"
    ok = subprocess.run([sys.executable, "-c", probe], cwd=tmp_path, capture_output=True, text=True)
    assert ok.returncode == 0, ok.stderr[-2000:]
    with open(tmp_path / "rank_gemm_unified_amd" / "csrc" / "k_pool.hip", "a") as f:
        f.write("\n// an edit after the build\n")
    bad = subprocess.run([sys.executable, "-c", probe], cwd=tmp_path, capture_output=True, text=True)
    assert bad.returncode != 0 and "stale" in bad.stderr, bad.stderr[-2000:]


def test_page_arithmetic_matches_worked_example(golden_dir):
    w = json.load(open(os.path.join(golden_dir, "slora_worked_example.json")))
    m, a = w["model"], w["adapter"]
    assert rg.lora_pool_pages_for(a["rank"], a["projections"], m["layers"]) == w["adapter_vectors_total"]
    assert rg.lora_pool_pages_for(a["rank"], a["projections"], 1) == w["adapter_vectors_per_layer"]
    assert rg.lora_kv_pages_per_token(m["layers"]) == w["kv_vectors_per_token"]
    for r in (0, 1, 8, 64, 128):
        for p in (1, 4):
            for L in (1, 32, 40):
                assert rg.lora_pool_pages_for(r, p, L) == adapter_page_count(r, L, p)
    assert rg.lora_pool_pages_for(-1, 4, 32) == -1 and rg.lora_kv_pages_per_token(-2) == -1
    assert rg.lora_kv_pages_per_token(40) == kv_pages_per_token(40)


def _bk_pool(num_pages, n_slots=1, max_adapters=16, max_rank=64, free_order=None):
    return rg.lora_pool_create(None, num_pages, 64, rg.LORA_BF16, max_rank, n_slots, max_adapters, None, free_order)


def _apply_c(pool, step, n_slots):
    op = step["op"]
    if op == "load":
        before = rg.lora_pool_free_list(pool)
        rc = rg.lora_pool_load_adapter(pool, step["aid"], step["rank"], None, None, stream=0, check=False)
        after = rg.lora_pool_free_list(pool)
        taken = []
        if rc == 0:
            pages, _, users = rg.lora_pool_adapter_pages(pool, step["aid"])
            taken = pages if users == 1 else []
        return rc, taken, (before, after)
    if op == "kv":
        r = rg.lora_pool_grow_kv(pool, step["rid"], step["layers"], check=False)
        return (r, [], None) if isinstance(r, int) else (0, r, None)
    if op == "free_kv":
        return rg.lora_pool_free_kv(pool, step["rid"], check=False), None, None
    if op == "release":
        return rg.lora_pool_release_adapter(pool, step["aid"], check=False), None, None
    if op == "evict":
        return rg.lora_pool_evict_adapter(pool, step["aid"], stream=0, check=False), None, None
    raise ValueError(op)


def test_hand_derived_trace_through_abi(golden_dir):
    traces = json.load(open(os.path.join(golden_dir, "pool_trace.json")))["traces"]
    for tr in traces:
        pool = _bk_pool(tr["num_pages"], tr["n_slots"], tr["max_adapters"], tr["max_rank"])
        try:
            for step in tr["steps"]:
                rc, taken, _ = _apply_c(pool, step, tr["n_slots"])
                assert rc == _STATUS[step["status"]], (step, rg.lora_last_error())
                if "pages" in step and step["status"] == "ok":
                    assert list(taken) == step["pages"], step
            fin = tr["final"]
            assert rg.lora_pool_free_list(pool) == fin["free"]
            assert rg.lora_pool_resident(pool) == fin["resident_in_load_order"]
            for rid, pages in fin["kv"].items():
                assert rg.lora_pool_kv_pages(pool, int(rid)) == pages
        finally:
            rg.lora_pool_free(pool)


def _model_status(s):
    return _STATUS[s]


def test_random_ops_match_model():
    rng = np.random.default_rng(1)
    for trial in range(30):
        n = int(rng.integers(8, 300))
        n_slots = int(rng.integers(1, 4))
        order = rng.permutation(n) if trial % 2 else None
        model = PagePoolModel(n, order)
        pool = _bk_pool(n, n_slots, max_adapters=10, max_rank=8, free_order=order)
        try:
            for _ in range(300):
                k = int(rng.integers(0, 5))
                aid, rid = int(rng.integers(0, 10)), int(rng.integers(0, 6))
                if k == 0:
                    rank = int(rng.integers(0, 9))
                    want = _model_status(model.admit(aid, rank, n_slots))
                    got = rg.lora_pool_load_adapter(pool, aid, rank, None, None, stream=0, check=False)
                elif k == 1:
                    layers = int(rng.integers(1, 4))
                    want = _model_status(model.add_kv_token(rid, layers))
                    r = rg.lora_pool_grow_kv(pool, rid, layers, check=False)
                    got = r if isinstance(r, int) else 0
                elif k == 2:
                    want = _model_status(model.end_request(rid))
                    got = rg.lora_pool_free_kv(pool, rid, check=False)
                elif k == 3:
                    want = _model_status(model.release(aid))
                    got = rg.lora_pool_release_adapter(pool, aid, check=False)
                else:
                    want = _model_status(model.evict(aid))
                    got = rg.lora_pool_evict_adapter(pool, aid, stream=0, check=False)
                assert got == want, (trial, k, rg.lora_last_error())
                assert rg.lora_pool_free_list(pool) == model.free_list
            assert rg.lora_pool_resident(pool) == model.resident_ids()
            for a, res in model.residents.items():
                got_pages, rank, users = rg.lora_pool_adapter_pages(pool, a)
                assert got_pages == res.pages and rank == res.rank and users == res.users
            st = rg.lora_pool_stats(pool)
            ms = model.stats()
            for key in ("num_pages", "free_pages", "kv_pages", "adapter_pages", "resident_adapters"):
                assert st[key] == ms[key], key
        finally:
            rg.lora_pool_free(pool)


_RULES = {"load_order": rg.LORA_VICTIM_LOAD_ORDER, "lru": rg.LORA_VICTIM_LRU, "farthest": rg.LORA_VICTIM_FARTHEST}


@pytest.mark.parametrize("victim", list(_RULES))
def test_victim_rules_match_model(victim):
    """Admission traffic that keeps the pool short of pages: the library's evictions under each
    victim rule (with a lookahead that changes as the trace goes on) match the pool model's."""
    rng = np.random.default_rng(11 + _RULES[victim])
    for trial in range(20):
        n_slots = int(rng.integers(1, 3))
        n = int(rng.integers(40, 160))
        model = PagePoolModel(n, victim=victim)
        pool = _bk_pool(n, n_slots, max_adapters=12, max_rank=8, free_order=None)
        try:
            assert rg.lora_pool_set_victim_rule(pool, _RULES[victim]) == 0
            ranks = rng.integers(1, 9, 12)
            held = []
            for step in range(200):
                if step % 7 == 0:
                    la = [int(a) for a in rng.integers(0, 12, int(rng.integers(0, 10)))]
                    model.set_lookahead(la)
                    rg.lora_pool_set_lookahead(pool, la)
                if held and rng.random() < 0.5:
                    a = held.pop(int(rng.integers(0, len(held))))
                    want, got = model.release(a), rg.lora_pool_release_adapter(pool, a, check=False)
                else:
                    a = int(rng.integers(0, 12))
                    want = model.admit(a, int(ranks[a]), n_slots)
                    got = rg.lora_pool_load_adapter(pool, a, int(ranks[a]), None, None, stream=0, check=False)
                    if want == "ok":
                        held.append(a)
                assert got == _model_status(want), (trial, step, rg.lora_last_error())
                assert rg.lora_pool_free_list(pool) == model.free_list
            assert rg.lora_pool_resident(pool) == model.resident_ids()
        finally:
            rg.lora_pool_free(pool)


def test_victim_rule_arguments():
    pool = _bk_pool(16, 1, max_adapters=4, max_rank=4, free_order=None)
    try:
        assert rg.lora_pool_set_victim_rule(pool, 3, check=False) == rg.LORA_EINVAL
        assert rg.lora_pool_set_lookahead(pool, [], check=False) == 0
        assert rg._lib.lora_pool_set_lookahead(pool, None, 2) == rg.LORA_EINVAL
        assert rg._lib.lora_pool_set_lookahead(pool, None, -1) == rg.LORA_EINVAL
        assert rg.lora_pool_set_victim_rule(None, 0, check=False) == rg.LORA_EINVAL
    finally:
        rg.lora_pool_free(pool)


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "many"])
def test_workload_plans_match_model(name):
    w = build(name)
    model = PagePoolModel(w.num_pages, w.free_order)
    want = model.run(w.ops, w.ranks, w.n_slots)
    pool = _bk_pool(w.num_pages, w.n_slots, w.max_adapters, 64, w.free_order)
    try:
        got = rg.run_pool_ops(pool, w.ops, w.ranks, lambda a: (None, None), stream=0)
        assert [_STATUS[s] for s in want] == got
        assert rg.lora_pool_free_list(pool) == model.free_list
        ids = model.resident_ids()
        for a in ids[:: max(1, len(ids) // 50)]:
            assert rg.lora_pool_adapter_pages(pool, a)[0] == model.pages_of(a)
    finally:
        rg.lora_pool_free(pool)


def test_error_codes():
    with pytest.raises(rg.LoraError) as e:
        rg.lora_pool_create(None, 10, 100, rg.LORA_BF16, 64, 1, 4, None)     # hidden not a multiple of 64
    assert e.value.code == rg.LORA_EINVAL
    with pytest.raises(rg.LoraError) as e:
        rg.lora_pool_create(None, 10, 64, 7, 64, 1, 4, None)
    assert e.value.code == rg.LORA_EINVAL
    with pytest.raises(rg.LoraError) as e:
        rg.lora_pool_create(None, 10, 64, rg.LORA_BF16, 65, 1, 4, None)
    assert e.value.code == rg.LORA_ERANK
    with pytest.raises(rg.LoraError) as e:
        rg.lora_pool_create(None, 4, 64, rg.LORA_BF16, 8, 1, 4, None, free_order=[0, 1, 1, 3])
    assert e.value.code == rg.LORA_EINVAL and "permutation" in str(e.value)
    with pytest.raises(rg.LoraError) as e:
        rg.lora_pool_create(None, 10, 64, rg.LORA_BF16, 8, 1, rg.LORA_MAX_ADAPTERS + 1, None)
    assert e.value.code == rg.LORA_EINVAL
    pool = _bk_pool(20, 1, 4, 8)
    try:
        assert rg.lora_pool_load_adapter(pool, 0, 9, None, None, 0, check=False) == rg.LORA_ERANK
        assert rg.lora_pool_load_adapter(pool, 4, 1, None, None, 0, check=False) == rg.LORA_EINVAL
        assert rg.lora_pool_load_adapter(pool, -1, 1, None, None, 0, check=False) == rg.LORA_EINVAL
        assert rg.lora_pool_load_adapter(pool, 0, 8, None, None, 0, check=False) == 0
        assert rg.lora_pool_load_adapter(pool, 1, 8, None, None, 0, check=False) == rg.LORA_ENOMEM
        assert rg.lora_pool_load_adapter(pool, 0, 4, None, None, 0, check=False) == rg.LORA_EEXIST
        assert rg.lora_pool_evict_adapter(pool, 0, 0, check=False) == rg.LORA_EBUSY
        assert rg.lora_pool_evict_adapter(pool, 2, 0, check=False) == rg.LORA_ENOENT
        assert rg.lora_pool_release_adapter(pool, 2, check=False) == rg.LORA_ENOENT
        assert rg.lora_pool_free_kv(pool, 5, check=False) == rg.LORA_ENOENT
        assert rg.lora_pool_grow_kv(pool, 0, 0, check=False) == rg.LORA_EINVAL
        assert len(rg.lora_pool_grow_kv(pool, 0, 2, check=False)) == 4
        assert rg.lora_pool_grow_kv(pool, 0, 1, check=False) == rg.LORA_ENOMEM
        with pytest.raises(rg.LoraError) as e:
            rg.lora_pool_page_table(pool, 0)
        assert e.value.code == rg.LORA_EINVAL
        # a projection on a bookkeeping-only pool is refused before any device work
        assert rg._lib.lora_project(pool, 16, 16, 16, 16, 16, 16, 4, 16, 256, 1 << 20, None) == rg.LORA_EINVAL
        assert rg._lib.lora_project(None, 16, 16, 16, 16, 16, 16, 4, 16, 256, 1 << 20, None) == rg.LORA_EINVAL
        # ... and so is a several-slot projection, with the slot count and slot range checked first
        ptrs = (ctypes.c_void_p * 5)(*([256] * 5))
        for n, slots, msg in ((0, [0], "n = 0"), (5, [0] * 5, "n = 5"), (1, [1], "slot 1"), (1, [-1], "slot -1"),
                              (1, [0], "bookkeeping-only")):
            sl = (ctypes.c_int32 * len(slots))(*slots)
            assert rg._lib.lora_project_slots(pool, n, sl, 256, ptrs, 16, 16, 16, 4, ptrs, 256, 1 << 20,
                                              None) == rg.LORA_EINVAL
            assert msg in rg.lora_last_error(), (msg, rg.lora_last_error())
        assert rg.lora_project_slots_workspace_size(pool, 0, 16) == 0
        assert rg.lora_project_workspace_size(pool, rg.LORA_MAX_TOKENS) > 0
        assert rg.lora_project_workspace_size(pool, rg.LORA_MAX_TOKENS + 1) == 0
        assert rg.lora_project_slots_workspace_size(pool, rg.LORA_MAX_CALL_SLOTS + 1, 16) == 0
        st = rg.lora_pool_stats(pool)
        assert st["adapter_pages"] == 16 and st["kv_pages"] == 4 and st["free_pages"] == 0
        assert st["loads"] == 1 and st["resident_adapters"] == 1
    finally:
        rg.lora_pool_free(pool)
    assert rg.lora_pool_free(None) == 0


def test_workspace_size_grows_with_tokens():
    pool = _bk_pool(100, 1, 32, 64)
    try:
        sizes = [rg.lora_project_workspace_size(pool, T) for T in (1, 16, 64, 256, 257, 4096)]
        assert all(s > 0 and s % 256 == 0 for s in sizes)
        assert sizes == sorted(sizes) or sizes[3] > sizes[4]     # decode keeps split-K partials
        assert rg.lora_project_workspace_size(pool, -1) == 0
    finally:
        rg.lora_pool_free(pool)
