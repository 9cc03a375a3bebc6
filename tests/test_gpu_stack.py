"""GPU parity of the Llama-13B-shaped stack at its configured size, on one GPU.

H = 5120, 40 layers x q/k/v/o = 160 slots, 1000 adapters of ranks U{8, 16, 32, 64} (each with A and B
on all 160 slots: about 91.6 GiB of pages), a pool of pages / 0.80 (about 114 GiB) fragmented by
seeded alloc/free churn with KV pages up to 15 % of it ("S-LoRA, in depth", section "Unified
paging": adapters and KV share one pool of H-vector pages).  One batch of 8448 rows: 4 prefill
requests of 2048 rows and 256 decode rows, Zipf(1.2) ids.  One step through the stack is 40 x (the
layer's q, k, v and o in one lora_project_slots_x call, o reading its own x); every slot's output
is kept.

Checked against the fp64 oracle: every row of 8 slots spread over the stack; on all 160 slots every
decode row and 64 seeded rows of each prefill request, with the per-token low-rank delta; the pages
the kernels read and the grouping they consume, bit for bit, on several slots; q/k/v/o in one call
equal to one call per slot, bit for bit; the fragmentation of the whole pool; KV pages unchanged."""
import time

import numpy as np
import pytest
import torch

import oracle
import rank_gemm_unified_amd as rg
from gpu_helpers import check_indices, errors, ids_ranks_scale, say
from workloads import build, storage_to_f64

pytestmark = pytest.mark.gpu

BF16_REL, BF16_ABS = 1e-2, 5e-2
FULL_SLOTS = (0, 3, 41, 62, 85, 118, 139, 159)      # every row checked: q, o, k, v, k, v, o, o
N_CANARY = 4096


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def stack():
    t0 = time.time()
    w = build("stack13b", device="cuda")
    assert w.n_slots == 160 and w.max_adapters == 1000 and w.T == 8448
    say(f"case stack13b full: H {w.hidden} T {w.T} slots {w.n_slots} pages {w.num_pages} "
        f"({w.num_pages * w.hidden * 2 / 2**30:.1f} GiB) ops {len(w.ops)}")
    pool = rg.Pool(w.num_pages, w.hidden, rg.LORA_BF16, n_slots=w.n_slots, max_adapters=w.max_adapters,
                   max_rank=w.max_rank, free_order=w.free_order)
    step = 20000
    for i in range(0, len(w.ops), step):
        st = pool.run_ops(w.ops[i:i + step], w.ranks, w.adapter_uncached)
        assert all(s == 0 for s in st), (i, rg.lora_last_error())
        torch.cuda.synchronize()
        say(f"  ops {min(i + step, len(w.ops))}/{len(w.ops)} at {time.time() - t0:.0f} s")
    stats = pool.stats()
    say("pool ready:", stats)
    # KV canaries: seeded bits in a sample of KV pages, checked after every projection of the step
    kv = []
    for rid in sorted({op[1] for op in w.ops if op[0] == "kv"}):
        try:
            kv.extend(rg.lora_pool_kv_pages(pool.handle, rid))
        except rg.LoraError:
            pass                                            # request freed by the churn
        if len(kv) >= 64 * N_CANARY:
            break
    rng = np.random.default_rng(1055)
    canary_pages = torch.as_tensor(rng.choice(np.array(kv, np.int64), N_CANARY, replace=False), device="cuda")
    canary = w.kv_canary(N_CANARY).view(torch.bfloat16)
    pool.pages[canary_pages] = canary
    # one step through the stack
    d_ids, d_ranks, d_scale = ids_ranks_scale(w)
    ys = [None] * w.n_slots
    for layer in range(w.n_slots // 4):   # q, k, v (layer input x) and o (x_o) in one call
        sl = list(range(4 * layer, 4 * layer + 4))
        ys[sl[0]:sl[0] + 4] = pool.project_slots(sl, [w.x_for_slot(s) for s in sl], [w.W(s) for s in sl],
                                                 d_ids, d_ranks, d_scale)
    torch.cuda.synchronize()
    assert rg.lora_check_device_errors(pool.handle, check=False) == 0, rg.lora_last_error()
    say(f"stack step done at {time.time() - t0:.0f} s")
    yield w, pool, ys, (canary_pages, canary)
    pool.close()
    w.drop_cache()
    del ys
    torch.cuda.empty_cache()


def _sample_rows(w):
    rng = np.random.default_rng(105)
    rows = [np.arange(w.T - 256, w.T)]                  # every decode row
    for start, n in w.segments:                          # 64 seeded rows of each prefill request
        rows.append(start + np.sort(rng.choice(n, 64, replace=False)))
    return np.concatenate(rows)


def _oracle_rows(w, slot, rows):
    """fp64 oracle on the given rows of one slot: (y, y with every token on no adapter)."""
    x64 = storage_to_f64(w.x_for_slot(slot)[torch.as_tensor(rows, device="cuda")])
    W64 = storage_to_f64(w.W(slot)).T
    ids = w.ids[rows]
    A, B = {}, {}
    for a in np.unique(ids):
        a = int(a)
        if a >= 0 and int(w.ranks[a]) > 0:
            at, b = w.adapter(a)
            A[a], B[a] = storage_to_f64(at[slot]).T, storage_to_f64(b[slot])
    ref = oracle.project(x64, W64, A, B, ids, w.scales)
    base = oracle.project(x64, W64, {}, {}, np.full(rows.size, -1), w.scales)
    return ref, base


def test_stack_pool_is_full_size_and_fragmented(stack):
    w, pool, _, _ = stack
    st = pool.stats()
    want_pages = int(sum(2 * int(r) * w.n_slots for r in w.ranks))
    assert st["resident_adapters"] == 1000 and st["adapter_pages"] == want_pages
    assert st["adapter_pages"] * w.hidden * 2 > 90 * 2**30               # about 91.6 GiB of adapter pages
    assert w.num_pages * w.hidden * 2 > 110 * 2**30 and st["kv_pages"] <= 0.16 * w.num_pages
    tab = pool.table.cpu().numpy()                                         # [160][1000][128]
    r2 = 2 * w.ranks.astype(np.int64)
    j = np.arange(tab.shape[2])
    live = j[None, None, :] < r2[None, :, None]
    pages = tab[np.broadcast_to(live, tab.shape)].astype(np.int64)
    assert pages.size == want_pages and pages.min() >= 0 and pages.max() < w.num_pages
    assert np.unique(pages).size == pages.size                             # pairwise distinct
    steps = np.broadcast_to(live[:, :, 1:], (tab.shape[0], tab.shape[1], tab.shape[2] - 1))
    adj = (np.abs(np.diff(tab.astype(np.int64), axis=2)) == 1) & steps
    say(f"stack13b full: {int(adj.sum())} of {int(steps.sum())} consecutive entries are neighbouring pages")
    assert adj.sum() <= 0.1 * steps.sum()


def test_stack_kv_pages_untouched(stack):
    _, pool, _, (pages, canary) = stack
    assert torch.equal(pool.pages[pages].view(torch.int16), canary.view(torch.int16))


@pytest.mark.parametrize("slot", [0, 3, 86, 159])
def test_stack_indices(stack, slot):
    w, pool, _, _ = stack
    say(f"indices slot {slot}:", check_indices(pool, w, slot))


def test_stack_all_rows_of_eight_slots(stack):
    w, pool, ys, _ = stack
    rows = np.arange(w.T)
    for slot in FULL_SLOTS:
        ref, _ = _oracle_rows(w, slot, rows)
        rel, mx = errors(ys[slot], ref)
        say(f"stack13b slot {slot}: all {w.T} rows, relL2={rel:.3e} maxabs={mx:.3e}")
        assert rel <= BF16_REL and mx <= BF16_ABS, slot


def test_stack_sampled_rows_all_slots(stack):
    """Every decode row and 64 seeded rows of each prefill request, on all 160 slots, against the
    oracle; plus each live token's low-rank delta (y minus the same slot's base-only run) within 10 %
    of the oracle's, and rows on no adapter equal to the base-only run bit for bit."""
    w, pool, ys, _ = stack
    rows = _sample_rows(w)
    sel = torch.as_tensor(rows, device="cuda")
    d_none, d_ranks, d_scale = ids_ranks_scale(w, np.full(w.T, -1, np.int32))
    ids = w.ids[rows]
    live = np.array([a >= 0 and w.ranks[a] > 0 for a in ids])
    worst = (0.0, 0.0, 0.0)
    for slot in range(w.n_slots):
        ref, base = _oracle_rows(w, slot, rows)
        rel, mx = errors(ys[slot][sel], ref)
        assert rel <= BF16_REL and mx <= BF16_ABS, (slot, rel, mx)
        y0 = pool.project(slot, w.x_for_slot(slot), w.W(slot), d_none, d_ranks, d_scale)
        d_gpu = storage_to_f64(ys[slot][sel]) - storage_to_f64(y0[sel])
        d_ref = ref - base
        rel_t = np.linalg.norm(d_gpu[live] - d_ref[live], axis=1) / np.linalg.norm(d_ref[live], axis=1)
        assert rel_t.max() <= 0.1, (slot, int(rows[live][rel_t.argmax()]), float(rel_t.max()))
        ident = sel[torch.as_tensor(np.nonzero(~live)[0], device="cuda")]
        assert torch.equal(ys[slot][ident].view(torch.int16), y0[ident].view(torch.int16)), slot
        worst = (max(worst[0], rel), max(worst[1], mx), max(worst[2], float(rel_t.max())))
        if slot % 40 == 39:
            say(f"  slots 0..{slot}: worst relL2 {worst[0]:.3e}, maxabs {worst[1]:.3e}, token delta {worst[2]:.3e}")
    say(f"stack13b: {rows.size} rows x {w.n_slots} slots checked")


@pytest.mark.parametrize("layer", [0, 21, 39])
def test_stack_qkvo_in_one_call_equals_per_slot(stack, layer):
    w, pool, ys, _ = stack
    d_ids, d_ranks, d_scale = ids_ranks_scale(w)
    for s in range(4 * layer, 4 * layer + 4):
        y1 = pool.project(s, w.x_for_slot(s), w.W(s), d_ids, d_ranks, d_scale)
        assert torch.equal(y1.view(torch.int16), ys[s].view(torch.int16)), s
