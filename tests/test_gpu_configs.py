"""GPU parity at full size of the many-adapter decode batch: H=4096, q/k/v/o of one layer, 2000
adapters plus a rank-0 identity adapter, 256 tokens with Zipf(1.0) ids (26 on the identity adapter),
a 60 %-KV pool of about 1.37 M pages (11 GB: page offsets beyond 4 GiB).

Every gather index the kernels use is compared bit for bit (lora_debug_project); outputs against the
fp64 oracle on every row, with the per-token low-rank delta; the q, k and v projections made by one
lora_project_slots call (which splits K into fewer ranges than a one-slot call) must agree with one
lora_project call per slot up to one bfloat16 rounding step, and two identical calls bit for bit.  The 13B-shaped
stack is checked at its configured size in test_gpu_stack.py."""
import numpy as np
import pytest
import torch

import rank_gemm_unified_amd as rg
from gpu_helpers import check_indices, device_pool, errors, ids_ranks_scale, oracle_y, run, say, within_one_rounding
from workloads import build, storage_to_f64

pytestmark = pytest.mark.gpu

BF16_REL, BF16_ABS = 1e-2, 5e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _gather_exact(w, pool, slot):
    """The pages the production kernels read for every token, and their grouping, bit for bit."""
    say(f"indices slot {slot}:", check_indices(pool, w, slot))


def _delta_check(w, pool, slot, y, ref, rows=None):
    """Per-token low-rank delta against the oracle's on the rows given: catches one token's wrong
    or missing adapter, which the global relative error would dilute.  Rows on no adapter or on a
    rank-0 adapter must equal the base-only run bit for bit."""
    rows = np.arange(w.T) if rows is None else rows
    none = np.full(w.T, -1, np.int32)
    y0 = run(pool, w, slot, ids=none)
    torch.cuda.synchronize()
    base = oracle_y(w, slot, rows=rows, ids=none)
    sel = torch.as_tensor(rows, device="cuda")
    d_gpu = storage_to_f64(y[sel]) - storage_to_f64(y0[sel])
    d_ref = ref - base
    ids = w.ids[rows]
    live = np.array([a >= 0 and w.ranks[a] > 0 for a in ids])
    rel_t = np.linalg.norm(d_gpu[live] - d_ref[live], axis=1) / np.linalg.norm(d_ref[live], axis=1)
    assert rel_t.max() <= 0.1, (int(rows[live][rel_t.argmax()]), float(rel_t.max()))
    ident = torch.as_tensor(rows[~live], device="cuda")
    assert torch.equal(y[ident].view(torch.int16), y0[ident].view(torch.int16))


# ---------------------------------------------------------------------------------------------
@pytest.fixture(scope="module")
def many():
    w = build("many", device="cuda")
    say("case many: H", w.hidden, "T", w.T, "slots", w.n_slots, "pages", w.num_pages)
    pool = device_pool(w)
    say("many: pool ready", pool.stats())
    yield w, pool
    pool.close()
    w.drop_cache()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("slot", [0, 1, 2, 3])
def test_many_adapters_parity(many, slot):
    w, pool = many
    say("case many slot", slot)
    assert w.num_pages * w.hidden * 2 > 2**32          # page offsets need 64 bits
    _gather_exact(w, pool, slot)
    y = run(pool, w, slot)
    torch.cuda.synchronize()
    assert rg.lora_check_device_errors(pool.handle, check=False) == 0, rg.lora_last_error()
    ref = oracle_y(w, slot)
    rel, mx = errors(y, ref)
    say(f"many slot {slot}: relL2={rel:.3e} maxabs={mx:.3e}")
    assert rel <= BF16_REL and mx <= BF16_ABS
    _delta_check(w, pool, slot, y, ref)


def test_many_adapters_qkv_in_one_call(many):
    w, pool = many
    say("case many: q/k/v in one call")
    d_ids, d_ranks, d_scale = ids_ranks_scale(w)
    ys = pool.project_slots([0, 1, 2], w.x_for_slot(0), [w.W(s) for s in (0, 1, 2)], d_ids, d_ranks, d_scale)
    again = pool.project_slots([0, 1, 2], w.x_for_slot(0), [w.W(s) for s in (0, 1, 2)], d_ids, d_ranks, d_scale)
    for s, y, y2 in zip((0, 1, 2), ys, again):
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), s
        assert within_one_rounding(y, run(pool, w, s)), s
    torch.cuda.synchronize()
    assert rg.lora_check_device_errors(pool.handle, check=False) == 0, rg.lora_last_error()
    rel, mx = errors(ys[1], oracle_y(w, 1))
    say(f"many q/k/v in one call, slot 1: relL2={rel:.3e} maxabs={mx:.3e}")
    assert rel <= BF16_REL and mx <= BF16_ABS
