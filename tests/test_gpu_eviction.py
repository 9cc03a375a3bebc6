"""Idle-adapter eviction on a device pool, under each victim rule.

"S-LoRA, in depth", section "Unified paging" and its pool sketch: a load that is short of pages first
reclaims idle adapters (no users) until enough pages are free; the victim rules (load order, least
recently admitted, farthest next request in a lookahead) follow the MoE-offload page ("Cache the
Experts You Will Need").  A full pool (KV pages plus resident adapters, no free page) takes loads of
new adapters that must reclaim idle ones.  Checked on the device, against the oracle's pool model
run on the same operations:
  * the library evicts the same adapters, in the same order, and hands out the same pages: the new
    adapters' pages are the reclaimed ones (the free list was empty);
  * the evicted adapters' page-table rows read -1 in every slot, and the new adapters' rows hold
    their pages;
  * KV pages keep their canary bits through the evictions, the loads (which scatter into reclaimed
    pages) and the projections;
  * projections whose tokens use surviving and new adapters match the fp64 oracle, and the pages
    the kernels read equal the table lookup bit for bit;
  * a load that cannot be satisfied even after reclaiming every idle adapter returns LORA_ENOMEM,
    and the adapters reclaimed on the way stay reclaimed (rows -1), as in the sketch."""
import numpy as np
import pytest
import torch

import oracle
import rank_gemm_unified_amd as rg
from gpu_helpers import check_indices, errors, ids_ranks_scale, oracle_y, say
from workloads import custom

pytestmark = pytest.mark.gpu

RULES = {"load_order": rg.LORA_VICTIM_LOAD_ORDER, "lru": rg.LORA_VICTIM_LRU, "farthest": rg.LORA_VICTIM_FARTHEST}
H, SLOTS, N_AD = 1024, 2, 12
STATUS = {"ok": 0, "enomem": rg.LORA_ENOMEM}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _full_pool(rule, seed, idle=(2, 3, 4, 5, 6, 7)):
    """Adapters 0..7 resident over two slots (2 and 5 admitted twice), the ones in `idle` finished,
    the rest still in use; KV pages fill the pool to fewer than 4 free pages.  The oracle's pool model
    runs the same operations."""
    rng = np.random.default_rng(seed)
    ranks = rng.choice([8, 16], N_AD).astype(np.int32)
    w = custom(H, ranks, np.zeros(4, np.int32), n_slots=SLOTS, device="cuda", seed=seed, load=[])
    resident = list(range(8))
    n = int(sum(2 * int(ranks[a]) * SLOTS for a in resident)) + 2 * 4 * 4 * 2
    order = rng.permutation(n).astype(np.int64)
    pool = rg.Pool(n, H, rg.LORA_BF16, n_slots=SLOTS, max_adapters=N_AD, free_order=order)
    model = oracle.PagePoolModel(n, order, victim=rule)
    assert rg.lora_pool_set_victim_rule(pool.handle, RULES[rule]) == 0
    for rid in range(4):
        for _ in range(4):
            rg.lora_pool_grow_kv(pool.handle, rid, 2)
            model.add_kv_token(rid, 2)
    for a in resident + [2, 5]:                          # 2 and 5 are admitted a second time
        at, b = w.adapter(a)
        rg.lora_pool_load_adapter(pool.handle, a, int(ranks[a]), at, b)
        assert model.admit(a, int(ranks[a]), SLOTS) == "ok"
    for a in idle:
        for _ in range(model.residents[a].users):
            assert rg.lora_pool_release_adapter(pool.handle, a) == 0
            assert model.release(a) == "ok"
    rid = 4
    while model.stats()["free_pages"] >= 4:              # the rest of the pool goes to KV
        rg.lora_pool_grow_kv(pool.handle, rid, 2)
        model.add_kv_token(rid, 2)
        rid += 1
    assert rg.lora_pool_free_list(pool.handle) == model.free_list
    kv = sorted(model.kv_page_set())                      # canary bits in every KV page
    canary = w.kv_canary(len(kv)).view(torch.bfloat16)
    kv_t = torch.as_tensor(kv, device="cuda")
    pool.pages[kv_t] = canary
    return w, pool, model, (kv_t, canary)


def _rows(pool, slot, a):
    return pool.table[slot, a].cpu().numpy()


@pytest.mark.parametrize("rule", list(RULES))
def test_loads_evict_idle_adapters_on_device(rule):
    w, pool, model, (kv_t, canary) = _full_pool(rule, seed=71 + RULES[rule])
    say(f"case eviction {rule}: pool {model.num_pages} pages, free {len(model.free_list)}, "
        f"victim order {model.eviction_order()}")
    if rule == "farthest":
        lookahead = [9, 3, 8, 6, 10]
        model.set_lookahead(lookahead)
        rg.lora_pool_set_lookahead(pool.handle, lookahead)
    evicted = []
    for a in (8, 9, 10):
        held = {b: list(model.pages_of(b)) for b in model.resident_ids()}
        free_before = list(model.free_list)
        st = model.admit(a, int(w.ranks[a]), SLOTS)
        assert st == "ok"
        at, b = w.adapter(a)
        assert rg.lora_pool_load_adapter(pool.handle, a, int(w.ranks[a]), at, b, check=False) == 0, rg.lora_last_error()
        gone = [g for g in held if g not in model.residents]
        short = len(free_before) < 2 * int(w.ranks[a]) * SLOTS
        assert bool(gone) == short, (a, gone, len(free_before))   # evicts exactly when pages are short
        evicted += gone
        assert rg.lora_pool_resident(pool.handle) == model.resident_ids()
        assert rg.lora_pool_free_list(pool.handle) == model.free_list
        pages, rank, users = rg.lora_pool_adapter_pages(pool.handle, a)
        assert pages == model.pages_of(a) and rank == int(w.ranks[a]) and users == 1
        reclaimed = set(free_before).union(*[held[g] for g in gone])
        assert set(pages) <= reclaimed                   # free pages, else pages of the adapters just evicted
        assert len(set(pages) - set(free_before)) >= len(pages) - len(free_before)
        say(f"  load {a} (rank {w.ranks[a]}): evicted {gone}")
    assert evicted, "the pool started full: the loads had to evict"
    torch.cuda.synchronize()
    # device page table: evicted rows are -1 in every slot, resident rows hold their page lists
    for a in range(N_AD):
        for s in range(SLOTS):
            row = _rows(pool, s, a)
            if a in model.residents:
                r = model.residents[a].rank
                assert row[: 2 * r].tolist() == model.pages_of(a)[2 * r * s: 2 * r * (s + 1)], (a, s)
                assert (row[2 * r:] == -1).all(), (a, s)
            else:
                assert (row == -1).all(), (a, s)
    # the new adapters' reclaimed pages hold their A columns and B rows
    for a in (8, 9, 10):
        at, b = w.adapter(a)
        r = int(w.ranks[a])
        for s in range(SLOTS):
            pids = torch.as_tensor(_rows(pool, s, a)[: 2 * r], device="cuda").long()
            assert torch.equal(pool.pages[pids[:r]].view(torch.int16), at[s].view(torch.int16))
            assert torch.equal(pool.pages[pids[r:]].view(torch.int16), b[s].view(torch.int16))
    # projections over the surviving and the new adapters, and tokens on no adapter
    rng = np.random.default_rng(5)
    ids = rng.choice(np.array(model.resident_ids() + [-1], np.int32), 96).astype(np.int32)
    w.ids, w.T = ids, int(ids.size)
    w.drop_cache("x")
    x = w.x()
    for s in range(SLOTS):
        d_ids, d_ranks, d_scale = ids_ranks_scale(w, ids)
        y = pool.project(s, x, w.W(s), d_ids, d_ranks, d_scale)
        torch.cuda.synchronize()
        assert rg.lora_check_device_errors(pool.handle, check=False) == 0, rg.lora_last_error()
        rel, mx = errors(y, oracle_y(w, s))
        say(f"  {rule} slot {s}: relL2={rel:.3e} maxabs={mx:.3e}, adapters {sorted(set(ids.tolist()))}")
        assert rel <= 1e-2 and mx <= 5e-2
        check_indices(pool, w, s, ids=ids, x=x)
    assert torch.equal(pool.pages[kv_t].view(torch.int16), canary.view(torch.int16)), "a KV page changed"
    pool.close()


def test_load_short_even_after_eviction_reports_enomem():
    w, pool, model, (kv_t, canary) = _full_pool("load_order", seed=90, idle=(3, 6))
    idle = model.eviction_order()
    assert idle == [3, 6]
    big = 11
    w.ranks[big] = 64                                     # needs more pages than the idle adapters hold
    assert 2 * 64 * SLOTS > len(model.free_list) + sum(len(model.pages_of(a)) for a in idle)
    assert model.admit(big, 64, SLOTS) == "enomem"
    at, b = w.adapter(big)
    assert rg.lora_pool_load_adapter(pool.handle, big, 64, at, b, check=False) == rg.LORA_ENOMEM
    assert rg.lora_pool_resident(pool.handle) == model.resident_ids() == [0, 1, 2, 4, 5, 7]
    assert rg.lora_pool_free_list(pool.handle) == model.free_list
    torch.cuda.synchronize()
    for a in idle:                                        # reclaimed on the way: rows cleared
        for s in range(SLOTS):
            assert (_rows(pool, s, a) == -1).all(), (a, s)
    assert torch.equal(pool.pages[kv_t].view(torch.int16), canary.view(torch.int16))
    pool.close()
