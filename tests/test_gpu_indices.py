"""The projection's own gather indices, bit for bit, on the GPU.

"S-LoRA, in depth", section "The architecture": the gather fetches each request's A and B pages from
wherever the pool placed them; section "Unified paging": a rank-r tensor is r pages.  The production
kernels, in their debug instantiations (lora_debug_project), record for every token the pages they
multiplied into its v and its y, and the grouping of tokens they consumed.  Those must equal the
oracle's table lookup (oracle.gather_page_ids) bit for bit, the grouping must be valid, and y must
equal lora_project's bit for bit.  Cases: the decode and prefill workloads, the float32 tiny workload,
and the path boundaries T = 1, 64, 65, 256, 257 (stream kernel, wide kernel, prefill path) with
identity and rank-0 tokens mixed in.  The many-adapter and 13B-shaped workloads are checked the same
way in test_gpu_configs.py and test_gpu_stack.py."""
import numpy as np
import pytest
import torch

from gpu_helpers import check_indices, device_pool, errors, oracle_y, run, say
from workloads import build, custom

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill"])
def test_workload_indices(name):
    w = build(name, device="cuda")
    say("case indices", name, "T", w.T)
    pool = device_pool(w)
    info = check_indices(pool, w, 0)
    say(name, info)
    pool.close()


@pytest.mark.parametrize("T", [1, 64, 65, 256, 257])
def test_path_boundary_indices(T):
    """32 adapters of ranks U{8, 16, 32, 64} plus a rank-0 adapter (id 32) at H = 4096; ids uniform
    over them and -1 (none)."""
    rng = np.random.default_rng(500 + T)
    ranks = [int(r) for r in rng.choice([8, 16, 32, 64], 32)] + [0]
    ids = rng.integers(-1, 33, T).astype(np.int32)
    w = custom(4096, ranks, ids, device="cuda", seed=600 + T)
    say("case indices at path boundary T", T)
    pool = device_pool(w)
    info = check_indices(pool, w, 0)
    say(T, info)
    pool.close()


def test_indices_one_adapter_and_no_adapter():
    """Degenerate groupings: every token on one adapter (one segment), and no token on any adapter."""
    for T in (64, 200, 600):
        w = custom(1024, [16, 64], np.ones(T, np.int32), device="cuda", seed=T)
        pool = device_pool(w)
        check_indices(pool, w, 0)
        check_indices(pool, w, 0, ids=np.full(T, -1, np.int32))
        pool.close()


@pytest.mark.parametrize("T", [40, 200])
def test_indices_ranks_at_quarter_boundaries(T):
    """Ranks on both sides of every quarter of j (1, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64) on the
    stream (T = 40) and wide (T = 200) decode kernels: the decode grouping orders segments by
    ceil(r / 16) and the finishing kernel skips quarters past every rank of its group of 8 tokens,
    so each class boundary must give the right pages, grouping and values."""
    ranks = [1, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64]
    rng = np.random.default_rng(700 + T)
    ids = rng.integers(-1, len(ranks), T).astype(np.int32)
    w = custom(1024, ranks, ids, device="cuda", seed=800 + T)
    say("case indices, ranks at quarter boundaries, T", T)
    pool = device_pool(w)
    info = check_indices(pool, w, 0)
    rel, mx = errors(run(pool, w, 0), oracle_y(w, 0))
    say(T, info, f"relL2={rel:.3e} maxabs={mx:.3e}")
    assert rel <= 1e-2 and mx <= 5e-2
    pool.close()
