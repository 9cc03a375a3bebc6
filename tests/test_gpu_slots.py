"""One call for several slots that share the tokens (the q, k and v projections of a layer, one x;
lora_project_slots_x: q, k, v and o, each slot with its own x): the outputs must equal, bit for bit,
what one lora_project call per slot gives on the decode T <= 64, prefill and float32 paths, and match
the fp64 oracle.  On the decode path for 64 < T <= 256 a call with several slots may split K into
fewer ranges than a one-slot call (the slots already fill the chip), so there the outputs must agree
with one call per slot up to one bfloat16 rounding step, and two identical calls bit for bit."""
import numpy as np
import pytest
import torch

import rank_gemm_unified_amd as rg
from gpu_helpers import device_pool, errors, ids_ranks_scale, oracle_y, say, within_one_rounding
from workloads import custom

pytestmark = pytest.mark.gpu

BF16_REL, BF16_ABS = 1e-2, 5e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("T,slots", [(48, [0, 1, 2]), (200, [0, 1, 2]), (700, [0, 1, 2]), (64, [2, 0]),
                                     (300, [1, 1, 3, 0]), (1, [3, 1]), (65, [0, 2]), (256, [1, 2, 3]),
                                     (257, [2, 1, 0])])
def test_slots_call_equals_one_call_per_slot(T, slots):
    rng = np.random.default_rng(T * 31 + len(slots))
    ranks = [8, 16, 32, 64, 0, 16, 8]
    if T > 256:   # prefill-shaped: runs of one adapter, a few single rows
        ids = np.repeat(rng.integers(-1, len(ranks), T // 50 + 1), 50)[:T].astype(np.int32)
        ids[rng.integers(0, T, 10)] = rng.integers(-1, len(ranks), 10)
    else:
        ids = rng.integers(-1, len(ranks), T).astype(np.int32)
    w = custom(1024, ranks, ids, n_slots=4, device="cuda", seed=900 + T)
    say(f"case slots T={T} slots={slots}")
    pool = device_pool(w)
    d_ids, d_ranks, d_scale = ids_ranks_scale(w)
    x = w.x(0)
    ys = pool.project_slots(slots, x, [w.W(s) for s in slots], d_ids, d_ranks, d_scale)
    again = pool.project_slots(slots, x, [w.W(s) for s in slots], d_ids, d_ranks, d_scale)
    singles = []
    for s in slots:
        y = torch.empty_like(x)
        pool.project(s, x, w.W(s), d_ids, d_ranks, d_scale, y=y)
        singles.append(y)
    torch.cuda.synchronize()
    assert rg.lora_check_device_errors(pool.handle, check=False) == 0, rg.lora_last_error()
    wide = 64 < T <= 256
    for s, y, y1, y2 in zip(slots, ys, singles, again):
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), s
        if wide:
            assert within_one_rounding(y, y1), s
        else:
            assert torch.equal(y.view(torch.int16), y1.view(torch.int16)), s
        rel, mx = errors(y, oracle_y(w, s, x=x))
        say(f"  slot {s}: relL2={rel:.3e} maxabs={mx:.3e}")
        assert rel <= BF16_REL and mx <= BF16_ABS
    pool.close()


@pytest.mark.parametrize("T,dtype", [(48, "bf16"), (200, "bf16"), (700, "bf16"), (257, "bf16"), (40, "f32")])
def test_slots_with_own_x_equal_one_call_per_slot(T, dtype):
    """q, k, v read x, o reads x_o: one lora_project_slots_x call for all four."""
    rng = np.random.default_rng(T * 7 + 1)
    ranks = [8, 16, 32, 64, 0, 16]
    ids = rng.integers(-1, len(ranks), T).astype(np.int32)
    if T > 256:
        ids = np.repeat(rng.integers(-1, len(ranks), T // 60 + 1), 60)[:T].astype(np.int32)
    w = custom(512, ranks, ids, n_slots=4, slot_x=[0, 0, 0, 1], n_x=2, dtype=dtype, device="cuda", seed=1200 + T)
    say(f"case slots with own x T={T} {dtype}")
    pool = device_pool(w)
    d_ids, d_ranks, d_scale = ids_ranks_scale(w)
    slots = [0, 1, 2, 3]
    xs = [w.x_for_slot(s) for s in slots]
    ys = pool.project_slots(slots, xs, [w.W(s) for s in slots], d_ids, d_ranks, d_scale)
    torch.cuda.synchronize()
    assert rg.lora_check_device_errors(pool.handle, check=False) == 0, rg.lora_last_error()
    bits = (lambda t: t.view(torch.int16)) if dtype == "bf16" else (lambda t: t.view(torch.int32))
    again = pool.project_slots(slots, xs, [w.W(s) for s in slots], d_ids, d_ranks, d_scale)
    wide = dtype == "bf16" and 64 < T <= 256
    for s, y, y2 in zip(slots, ys, again):
        y1 = pool.project(s, xs[s], w.W(s), d_ids, d_ranks, d_scale)
        assert torch.equal(bits(y), bits(y2)), s
        if wide:
            assert within_one_rounding(y, y1), s
        else:
            assert torch.equal(bits(y), bits(y1)), s
        rel, mx = errors(y, oracle_y(w, s))
        say(f"  slot {s}: relL2={rel:.3e} maxabs={mx:.3e}")
        assert rel <= (BF16_REL if dtype == "bf16" else 1e-4) and (dtype != "bf16" or mx <= BF16_ABS)
    # an output over another slot's input is refused before any device work
    ws = torch.empty(rg.lora_project_slots_workspace_size(pool.handle, 2, w.T), dtype=torch.uint8, device="cuda")
    x0, x1 = xs[0].clone(), xs[3].clone()
    rc = rg.lora_project_slots_x(pool.handle, [0, 3], [x0, x1], [w.W(0), w.W(3)], d_ids, d_ranks, d_scale, w.T,
                                 [torch.empty_like(x0), x1], ws, check=False)
    assert rc == rg.LORA_EINVAL and "overlaps" in rg.lora_last_error()
    assert torch.equal(x1, xs[3])
    pool.close()


def test_slots_call_rejects_bad_arguments():
    w = custom(256, [8, 16], np.array([0, 1, -1, 0], np.int32), n_slots=2, device="cuda", seed=3)
    pool = device_pool(w)
    d_ids, d_ranks, d_scale = ids_ranks_scale(w)
    x = w.x(0)
    ws = torch.empty(rg.lora_project_slots_workspace_size(pool.handle, 2, w.T), dtype=torch.uint8, device="cuda")
    y0, y1 = torch.full_like(x, 7.0), torch.full_like(x, 7.0)
    args = (x, [w.W(0), w.W(1)], d_ids, d_ranks, d_scale, w.T)
    assert rg.lora_project_slots(pool.handle, [0, 2], *args, [y0, y1], ws, check=False) == rg.LORA_EINVAL
    assert rg.lora_project_slots(pool.handle, [0, 1], *args, [y0, y0], ws, check=False) == rg.LORA_EINVAL
    assert rg.lora_project_slots(pool.handle, [0, 1], *args, [y0, y1], ws, workspace_bytes=ws.numel() - 256,
                                 check=False) == rg.LORA_EINVAL
    assert rg.lora_project_slots(pool.handle, [0] * 5, x, [w.W(0)] * 5, d_ids, d_ranks, d_scale, w.T, [y0] * 5,
                                 ws, check=False) == rg.LORA_EINVAL
    torch.cuda.synchronize()
    assert bool((y0 == 7.0).all()) and bool((y1 == 7.0).all())   # nothing ran
    pool.close()


def test_slots_call_float32_pool():
    """The float32 pool runs the slots one after another: same bits as one call per slot, every
    output within the float32 bound of the oracle, and overlapping outputs refused before any work."""
    rng = np.random.default_rng(77)
    ranks = [8, 16, 4, 0]
    ids = rng.integers(-1, len(ranks), 40).astype(np.int32)
    w = custom(256, ranks, ids, dtype="f32", n_slots=3, device="cuda", seed=78)
    say("case slots float32 T=40 slots=[2, 0, 1]")
    pool = device_pool(w)
    d_ids, d_ranks, d_scale = ids_ranks_scale(w)
    x = w.x(0)
    slots = [2, 0, 1]
    ys = pool.project_slots(slots, x, [w.W(s) for s in slots], d_ids, d_ranks, d_scale)
    for s, y in zip(slots, ys):
        y1 = pool.project(s, x, w.W(s), d_ids, d_ranks, d_scale)
        assert torch.equal(y, y1), s
        rel, mx = errors(y, oracle_y(w, s, x=x))
        assert rel <= 1e-4, (s, rel)
    ws = torch.empty(rg.lora_project_slots_workspace_size(pool.handle, 2, w.T), dtype=torch.uint8, device="cuda")
    y0 = torch.full_like(x, 7.0)
    assert rg.lora_project_slots(pool.handle, [0, 1], x, [w.W(0), w.W(1)], d_ids, d_ranks, d_scale, w.T,
                                 [y0, y0[1:]], ws, check=False) == rg.LORA_EINVAL
    torch.cuda.synchronize()
    assert rg.lora_check_device_errors(pool.handle, check=False) == 0, rg.lora_last_error()
    assert bool((y0 == 7.0).all())
    pool.close()


@pytest.mark.parametrize("T", [48, 300])   # decode path (grouping per slot) and prefill path (shared)
def test_slots_call_bad_row_in_one_slot(T):
    """A page id out of range in slot 1's row of adapter 1 is reported as a device error, and that
    adapter's tokens get the base product only: in slot 1 on the decode path, in every slot of the
    call on the prefill path (whose one grouping serves all slots)."""
    rng = np.random.default_rng(5 + T)
    ranks = [8, 16, 32]
    ids = rng.integers(0, len(ranks), T).astype(np.int32)
    w = custom(512, ranks, ids, n_slots=2, device="cuda", seed=40 + T)
    say(f"case slots bad row T={T}")
    pool = device_pool(w)
    pool.table[1][1, 0] = w.num_pages + 5
    d_ids, d_ranks, d_scale = ids_ranks_scale(w)
    x = w.x(0)
    ys = pool.project_slots([0, 1], x, [w.W(0), w.W(1)], d_ids, d_ranks, d_scale)
    torch.cuda.synchronize()
    assert rg.lora_check_device_errors(pool.handle, check=False) == rg.LORA_EDEVICE
    off = np.where(ids == 1, -1, ids).astype(np.int32)
    for s, y in zip((0, 1), ys):
        want_ids = off if (s == 1 or T > 256) else ids
        rel, mx = errors(y, oracle_y(w, s, x=x, ids=want_ids))
        say(f"  slot {s}: relL2={rel:.3e} maxabs={mx:.3e}")
        assert rel <= BF16_REL and mx <= BF16_ABS
    pool.close()


def test_slots_call_with_no_tokens():
    """T = 0: the call succeeds and writes nothing."""
    w = custom(256, [8, 16], np.array([0, 1, -1, 0], np.int32), n_slots=2, device="cuda", seed=4)
    pool = device_pool(w)
    d_ids, d_ranks, d_scale = ids_ranks_scale(w)
    x = w.x(0)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    y0, y1 = torch.full_like(x, 7.0), torch.full_like(x, 7.0)
    assert rg.lora_project_slots(pool.handle, [0, 1], x, [w.W(0), w.W(1)], d_ids, d_ranks, d_scale, 0, [y0, y1],
                                 ws, check=False) == rg.LORA_OK
    torch.cuda.synchronize()
    assert bool((y0 == 7.0).all()) and bool((y1 == 7.0).all())
    pool.close()
