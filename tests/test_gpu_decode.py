"""GPU parity of the decode-shaped path (T <= 256) and the float32 path against the fp64 oracle,
plus the bit-exact gather and pool-content checks and the bitwise invariants."""
import numpy as np
import pytest
import torch

import oracle
import rank_gemm_unified_amd as rg
from gpu_helpers import (bf16_round_f64, check_indices, device_pool, errors, ids_ranks_scale, oracle_y, run, say,
                         within_one_rounding)
from workloads import build, custom, storage_to_f64

pytestmark = pytest.mark.gpu

BF16_REL, BF16_ABS, F32_REL = 1e-2, 5e-2, 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    say("gpu:", torch.cuda.get_device_name(0))


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _pool_contents_exact(pool, w):
    """Every resident adapter's pages hold its A columns and B rows bit for bit, in the order the
    oracle's expected_page_rows defines (page j < r: column j of A; page r + j: row j of B)."""
    table = pool.table.cpu().numpy()
    for a in w.loaded_adapters():
        r = int(w.ranks[a])
        if r == 0:
            continue
        at, b = w.adapter(a)
        for slot in range(w.n_slots):
            rows = oracle.expected_page_rows(table[slot], a, r, _bits(at[slot]).cpu().numpy(),
                                             _bits(b[slot]).cpu().numpy())
            pids = torch.as_tensor([p for p, _ in rows], device=pool.pages.device).long()
            want = np.stack([v for _, v in rows])
            assert np.array_equal(_bits(pool.pages[pids]).cpu().numpy(), want), (a, slot)


def test_tiny_f32_parity():
    w = build("tiny", device="cuda")
    say("case tiny f32", w.hidden, w.T)
    pool = device_pool(w)
    _pool_contents_exact(pool, w)
    y = run(pool, w, 0)
    torch.cuda.synchronize()
    assert rg.lora_check_device_errors(pool.handle, check=False) == 0
    rel, mx = errors(y, oracle_y(w, 0))
    say(f"tiny relL2={rel:.3e} maxabs={mx:.3e}")
    assert rel <= F32_REL


def test_decode_parity_and_gather():
    w = build("decode", device="cuda")
    say("case decode bf16", w.hidden, w.T)
    pool = device_pool(w)
    _pool_contents_exact(pool, w)
    ids, ranks, _ = ids_ranks_scale(w)
    out = torch.empty((w.T, 2 * w.max_rank), dtype=torch.int32, device="cuda")
    rg.lora_debug_gather(pool.handle, pool.table[0], ids, ranks, w.T, out)   # the table view
    want = oracle.gather_page_ids(pool.table[0].cpu().numpy(), w.ids, w.ranks, w.max_rank)
    assert np.array_equal(out.cpu().numpy(), want)
    check_indices(pool, w, 0)                                                  # the kernels' own indices
    y = run(pool, w, 0)
    torch.cuda.synchronize()
    assert rg.lora_check_device_errors(pool.handle, check=False) == 0
    ref = oracle_y(w, 0)
    rel, mx = errors(y, ref)
    say(f"decode relL2={rel:.3e} maxabs={mx:.3e}")
    assert rel <= BF16_REL and mx <= BF16_ABS
    # per-token low-rank delta: catches a single token's wrong or missing adapter
    y0 = run(pool, w, 0, ids=np.full(w.T, -1, np.int32))
    base = oracle_y(w, 0, ids=np.full(w.T, -1, np.int32))
    d_gpu = storage_to_f64(y) - storage_to_f64(y0)
    d_ref = ref - base
    for t in range(w.T):
        rel_t = np.linalg.norm(d_gpu[t] - d_ref[t]) / np.linalg.norm(d_ref[t])
        assert rel_t <= 0.1, (t, rel_t)


@pytest.mark.parametrize("T", [1, 5, 16, 37, 64, 100, 128, 200, 256])
def test_decode_shapes_integer_exact(T):
    """Integer-valued inputs: every partial sum is exact in float32, so the output must equal the
    oracle's exact result rounded once to bfloat16, bit for bit."""
    rng = np.random.default_rng(T)
    ranks = [4, 1, 0, 3, 2]
    ids = rng.integers(-1, len(ranks), T)
    w = custom(128, ranks, ids, values="int", scales=[2, 1, 1, 2, 1], device="cuda", seed=T)
    say("case int-exact T", T)
    pool = device_pool(w)
    y = run(pool, w, 0)
    torch.cuda.synchronize()
    ref = oracle_y(w, 0)
    assert np.all(ref == np.round(ref)) and np.abs(ref).max() < 2 ** 24
    assert torch.equal(y.cpu().view(torch.int16), bf16_round_f64(ref).view(torch.int16))


def test_decode_wide_multipass_integer_exact():
    """The T > 64 kernel deals its shrink work units (adapter segment, 16 pages, 16 tokens) over the
    waves of all its workgroups; at H = 128 one pass holds 16 units, so 40 adapters of ranks 1..64
    over 200 tokens take several passes over K.  Integer-valued inputs: the output must equal the
    oracle's exact result rounded once, bit for bit."""
    rng = np.random.default_rng(40)
    ranks = [int(r) for r in rng.integers(1, 65, 40)]
    ids = rng.integers(-1, 40, 200)
    w = custom(128, ranks, ids, values="int", scales=[1] * 40, device="cuda", seed=40)
    say("case wide multipass: 40 adapters, T", w.T)
    pool = device_pool(w)
    y = run(pool, w, 0)
    torch.cuda.synchronize()
    assert rg.lora_check_device_errors(pool.handle, check=False) == 0
    ref = oracle_y(w, 0)
    assert np.all(ref == np.round(ref)) and np.abs(ref).max() < 2 ** 24
    assert torch.equal(y.cpu().view(torch.int16), bf16_round_f64(ref).view(torch.int16))


# (H, T): every K-steps-per-wave variant of the T <= 64 kernel (1, 2, 4, 8), 16-row blocks 1..4,
# waves with no K steps (H = 64), ragged quarters (192), a split count that is not a divisor of 8
# (5120: plain workgroup order) and the largest hidden size the kernel takes (8192, 1024 workgroups)
@pytest.mark.parametrize("H,T", [(64, 48), (192, 48), (512, 48), (5120, 48), (3072, 30), (2048, 64),
                                 (8192, 64), (1024, 7)])
def test_decode_hidden_sizes(H, T):
    rng = np.random.default_rng(H)
    ranks = [8, 16, 64, 0, 32]
    ids = rng.integers(-1, len(ranks), T)
    w = custom(H, ranks, ids, device="cuda", seed=H)
    say("case hidden", H, "T", T)
    pool = device_pool(w)
    y = run(pool, w, 0)
    torch.cuda.synchronize()
    rel, mx = errors(y, oracle_y(w, 0))
    say(f"H={H} relL2={rel:.3e} maxabs={mx:.3e}")
    assert rel <= BF16_REL and mx <= BF16_ABS


@pytest.mark.parametrize("T", [48, 200])   # the T <= 64 kernel and the T > 64 kernel
def test_token_order_and_relabelling_bitwise(T):
    """A token's result depends only on its own x and its adapter.  Permuting the tokens permutes the
    rows of y; naming the adapters differently (each one's weights, rank and scale moved to its new
    id) changes nothing.  Both bit for bit."""
    rng = np.random.default_rng(1000 + T)
    ranks = [8, 16, 64, 0, 32, 8, 16]
    ids = rng.integers(-1, len(ranks), T).astype(np.int32)
    w = custom(512, ranks, ids, device="cuda", seed=1000 + T)
    say("case order/relabel T", T)
    pool = device_pool(w)
    y = run(pool, w, 0)
    perm = rng.permutation(T)
    dperm = torch.as_tensor(perm, device="cuda")
    yp = run(pool, w, 0, ids=ids[perm], x=w.x()[dperm])
    # the same adapters under other ids, in a fresh pool
    sigma = rng.permutation(len(ranks))
    pool2 = rg.Pool(w.num_pages, w.hidden, rg.LORA_BF16, n_slots=1, max_adapters=len(ranks),
                    max_rank=w.max_rank, free_order=w.free_order)
    ranks2 = np.zeros(len(ranks), np.int32)
    scales2 = np.zeros(len(ranks), np.float32)
    for a in range(len(ranks)):
        ranks2[sigma[a]] = ranks[a]
        scales2[sigma[a]] = w.scales[a]
        at, b = w.adapter(a) if ranks[a] > 0 else (None, None)
        rg.lora_pool_load_adapter(pool2.handle, int(sigma[a]), int(ranks[a]), at, b)
    ids2 = np.where(ids >= 0, sigma[np.maximum(ids, 0)], -1).astype(np.int32)
    y2 = torch.empty_like(y)
    pool2.project(0, w.x(), w.W(0), torch.as_tensor(ids2, device="cuda"), torch.as_tensor(ranks2, device="cuda"),
                  torch.as_tensor(scales2, device="cuda"), y=y2)
    torch.cuda.synchronize()
    assert rg.lora_check_device_errors(pool2.handle, check=False) == 0
    assert torch.equal(yp.view(torch.int16), y[dperm].view(torch.int16))
    assert torch.equal(y2.view(torch.int16), y.view(torch.int16))
    pool2.close()


def test_identity_rows_bitwise():
    w = build("decode", device="cuda")
    pool = device_pool(w)
    ids = w.ids.copy()
    ids[::3] = -1
    y = run(pool, w, 0, ids=ids)
    y0 = run(pool, w, 0, ids=np.full(w.T, -1, np.int32))
    torch.cuda.synchronize()
    assert torch.equal(y[::3].view(torch.int16), y0[::3].view(torch.int16))
    ref = oracle_y(w, 0, ids=np.full(w.T, -1, np.int32))
    rel, mx = errors(y0, ref)
    assert rel <= BF16_REL and mx <= BF16_ABS


def test_placement_and_scaling_invariance():
    """Reloading the adapters into different pages, and scaling x by 2^k, change nothing but the
    exact power of two."""
    w = build("decode", device="cuda")
    pool = device_pool(w)
    y1 = run(pool, w, 0)
    used = sorted(set(int(a) for a in w.ids))
    before = {a: rg.lora_pool_adapter_pages(pool.handle, a)[0] for a in used}
    for a in used:
        rg.lora_pool_release_adapter(pool.handle, a)
        rg.lora_pool_evict_adapter(pool.handle, a)
    for i in range(8):      # shift the free list so the reloads land elsewhere
        assert isinstance(rg.lora_pool_grow_kv(pool.handle, 10 ** 6 + i, 1), list)
    for a in used[::-1]:
        at, b = w.adapter(a)
        rg.lora_pool_load_adapter(pool.handle, a, int(w.ranks[a]), at, b)
    after = {a: rg.lora_pool_adapter_pages(pool.handle, a)[0] for a in used}
    assert all(before[a] != after[a] for a in used)
    y2 = run(pool, w, 0)
    y4 = run(pool, w, 0, x=w.x() * 4)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal((y1.float() * 4).to(torch.bfloat16).view(torch.int16), y4.view(torch.int16))


def test_kv_pages_untouched():
    w = build("decode", device="cuda")
    pool = device_pool(w)
    rids = sorted({op[1] for op in w.ops if op[0] == "kv"})
    kv = sorted(p for rid in rids for p in rg.lora_pool_kv_pages(pool.handle, rid))
    assert len(kv) > 0.5 * w.num_pages
    idx = torch.as_tensor(kv, device="cuda").long()
    canary = w.kv_canary(len(kv)).view(torch.bfloat16)
    pool.pages[idx] = canary
    before = pool.pages[idx].clone()
    run(pool, w, 0)
    at, b = w.adapter(0)
    rg.lora_pool_release_adapter(pool.handle, 0)
    rg.lora_pool_evict_adapter(pool.handle, 0)
    rg.lora_pool_load_adapter(pool.handle, 0, int(w.ranks[0]), at, b)
    run(pool, w, 0)
    torch.cuda.synchronize()
    assert torch.equal(pool.pages[idx].view(torch.int16), before.view(torch.int16))


def test_two_streams_isolated():
    """Two batches with disjoint adapters, launched interleaved on two streams, each equal their
    single-stream results bitwise (no shared 'active adapter')."""
    w = build("decode", device="cuda")
    pool = device_pool(w)
    ids_a = np.where(w.ids % 2 == 0, w.ids, -1).astype(np.int32)
    ids_b = np.where(w.ids % 2 == 1, w.ids, -1).astype(np.int32)
    ref_a, ref_b = run(pool, w, 0, ids=ids_a), run(pool, w, 0, ids=ids_b)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        for ids, s in ((ids_a, s1), (ids_b, s2)):
            with torch.cuda.stream(s):
                d_ids, d_ranks, d_scale = ids_ranks_scale(w, ids)
                y = torch.empty_like(w.x())
                ws = torch.empty(rg.lora_project_workspace_size(pool.handle, w.T), dtype=torch.uint8, device="cuda")
                rg.lora_project(pool.handle, w.x(), w.W(0), pool.table[0], d_ids, d_ranks, d_scale, w.T, y, ws,
                                stream=s)
                outs.append((y, ws, d_ids, d_ranks, d_scale, ids is ids_a))
    torch.cuda.synchronize()
    for y, *_, is_a in outs:
        assert torch.equal(y.view(torch.int16), (ref_a if is_a else ref_b).view(torch.int16))


def test_device_checks_flag_bad_tokens():
    """Out-of-range ids, wrong ranks and unloaded adapters are caught on the device: those tokens
    get the base product and the error word reports them."""
    w = build("decode", device="cuda")
    pool = device_pool(w)
    assert rg.lora_check_device_errors(pool.handle, check=False) == 0
    ids = w.ids.copy()
    ids[0] = 5000            # out of range
    ranks = w.ranks.copy()
    a_bad = int(ids[1])
    ranks[a_bad] = ranks[a_bad] // 2   # not the loaded rank
    d_ids = torch.as_tensor(ids, device="cuda")
    y = torch.empty_like(w.x())
    ws = pool.workspace(w.T)
    rg.lora_project(pool.handle, w.x(), w.W(0), pool.table[0], d_ids, torch.as_tensor(ranks, device="cuda"),
                    torch.as_tensor(w.scales, device="cuda"), w.T, y, ws)
    rc = rg.lora_check_device_errors(pool.handle, check=False)
    assert rc == rg.LORA_EDEVICE
    msg = rg.lora_last_error()
    assert "adapter-id-out-of-range" in msg and "adapter-not-loaded-at-this-rank" in msg
    assert rg.lora_check_device_errors(pool.handle, check=False) == 0     # cleared
    bad = (ids == 5000) | (ids == a_bad)
    y0 = run(pool, w, 0, ids=np.full(w.T, -1, np.int32))
    torch.cuda.synchronize()
    assert torch.equal(y[torch.as_tensor(bad, device="cuda")].view(torch.int16),
                       y0[torch.as_tensor(bad, device="cuda")].view(torch.int16))


def test_host_validation_touches_nothing():
    w = build("tiny", device="cuda")
    pool = device_pool(w)
    d_ids, d_ranks, d_scale = ids_ranks_scale(w)
    y = torch.full_like(w.x(), 7.0)
    ws = pool.workspace(w.T)
    rc = rg.lora_project(pool.handle, w.x(), w.W(0), pool.table[0], d_ids, d_ranks, d_scale, w.T, y, ws,
                         workspace_bytes=16, check=False)
    assert rc == rg.LORA_EINVAL
    rc = rg.lora_project(pool.handle, w.x(), w.W(0), pool.table[0], d_ids, d_ranks, d_scale, w.T, w.x(), ws,
                         check=False)
    assert rc == rg.LORA_EINVAL        # y overlaps x
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
    assert rg.lora_project(pool.handle, w.x(), w.W(0), pool.table[0], d_ids, d_ranks, d_scale, 0, y, ws) == 0


# (H, T) on the T > 64 kernel: one column tile (64), ragged quarters (192), a split count that is not
# a divisor of 8 (5120: three splits, uneven K ranges), two splits (8192) and the smallest T (65);
# each also as one call for three slots (fewer K splits per slot)
@pytest.mark.parametrize("H,T", [(64, 100), (192, 130), (3072, 65), (5120, 200), (8192, 256)])
def test_decode_wide_hidden_sizes(H, T):
    rng = np.random.default_rng(H + T)
    ranks = [8, 16, 64, 0, 32, 1, 48]
    ids = rng.integers(-1, len(ranks), T)
    w = custom(H, ranks, ids, n_slots=3, device="cuda", seed=H + T)
    say("case wide hidden", H, "T", T)
    pool = device_pool(w)
    d_ids, d_ranks, d_scale = ids_ranks_scale(w)
    x = w.x(0)
    ys = pool.project_slots([0, 1, 2], x, [w.W(s) for s in range(3)], d_ids, d_ranks, d_scale)
    again = pool.project_slots([0, 1, 2], x, [w.W(s) for s in range(3)], d_ids, d_ranks, d_scale)
    for s in range(3):
        y1 = pool.project(s, x, w.W(s), d_ids, d_ranks, d_scale)
        torch.cuda.synchronize()
        assert rg.lora_check_device_errors(pool.handle, check=False) == 0, rg.lora_last_error()
        ref = oracle_y(w, s, x=x)
        for y in (y1, ys[s]):
            rel, mx = errors(y, ref)
            assert rel <= BF16_REL and mx <= BF16_ABS, (s, rel, mx)
        assert torch.equal(ys[s].view(torch.int16), again[s].view(torch.int16)), s
        assert within_one_rounding(ys[s], y1), s
    say(f"H={H} T={T}: 3 slots, one call and one call per slot")
    pool.close()
