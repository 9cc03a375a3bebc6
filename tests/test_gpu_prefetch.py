"""Adapter loads from pinned host memory on a copy stream while projections run on the compute stream
("S-LoRA, in depth", section "Scheduling: prefetch, clustering and early abort": the next batch's
adapters are copied while the current batch computes; pinned memory and a separate copy stream make
the overlap possible).  The compute stream waits on the copy's event before the first projection
that uses the new adapters; every output must match the fp64 oracle."""
import numpy as np
import pytest
import torch

import rank_gemm_unified_amd as rg
from gpu_helpers import device_pool, errors, ids_ranks_scale, oracle_y, say
from workloads import custom

pytestmark = pytest.mark.gpu

BF16_REL, BF16_ABS = 1e-2, 5e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _pinned(t):
    """A new pinned host tensor holding t's values (pinned memory is allocated, never registered)."""
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t.cpu())
    return h


def _project(pool, w, ids, stream):
    d_ids, d_ranks, d_scale = ids_ranks_scale(w, ids)
    x = w.x_for_slot(0)
    y = torch.empty_like(x)
    pool.project(0, x, w.W(0), d_ids, d_ranks, d_scale, y=y, stream=stream)
    return y


@pytest.mark.parametrize("T", [40, 200])   # the T <= 64 kernel and the T > 64 kernel
def test_loads_on_a_copy_stream_overlap_projections(T):
    rng = np.random.default_rng(31 + T)
    ranks = [8, 16, 32, 64, 16, 8, 64]
    late = [3, 4, 5, 6]                                   # evicted, then reloaded on the copy stream
    ids_old = rng.integers(-1, 3, T).astype(np.int32)    # adapters 0..2 (and identity rows)
    ids_new = rng.integers(-1, len(ranks), T).astype(np.int32)
    w = custom(1024, ranks, ids_new, device="cuda", seed=500 + T)
    pool = device_pool(w)                                 # every adapter resident, one user each
    host = {a: tuple(_pinned(t) for t in w.adapter(a)) for a in late}
    comp = torch.cuda.current_stream()
    copy = torch.cuda.Stream()                            # default priority
    for a in late:
        rg.lora_pool_release_adapter(pool.handle, a)
        rg.lora_pool_evict_adapter(pool.handle, a, stream=comp)
    torch.cuda.synchronize()
    loads0 = pool.stats()["loads"]
    say(f"case prefetch T={T}: {len(late)} adapters reloaded from pinned host memory on a copy stream")

    ys_old = [_project(pool, w, ids_old, comp) for _ in range(6)]   # queued on the compute stream
    for a in late:                                                    # meanwhile, on the copy stream
        at, b = host[a]
        rg.lora_pool_load_adapter(pool.handle, a, int(ranks[a]), at, b, stream=copy)
    done = torch.cuda.Event()
    done.record(copy)
    comp.wait_event(done)
    y_new = _project(pool, w, ids_new, comp)
    ys_old.append(_project(pool, w, ids_old, comp))
    torch.cuda.synchronize()
    assert rg.lora_check_device_errors(pool.handle, check=False) == 0, rg.lora_last_error()

    ref_old, ref_new = oracle_y(w, 0, ids=ids_old), oracle_y(w, 0, ids=ids_new)
    for y in ys_old:
        rel, mx = errors(y, ref_old)
        assert rel <= BF16_REL and mx <= BF16_ABS, (rel, mx)
        assert torch.equal(y.view(torch.int16), ys_old[0].view(torch.int16))   # same inputs, same bits
    rel, mx = errors(y_new, ref_new)
    say(f"T={T}: after the copy relL2={rel:.3e} maxabs={mx:.3e}")
    assert rel <= BF16_REL and mx <= BF16_ABS
    st = pool.stats()
    assert st["loads"] == loads0 + len(late) and st["resident_adapters"] == len(ranks), st
    pool.close()
