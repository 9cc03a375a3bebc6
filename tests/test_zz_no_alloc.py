"""lora_project_noalloc (the entry point for callers that cannot allocate) against lora_project.

The two run the same kernels; the only difference is where the workspace lives (the library's
per-GPU scratch array instead of a caller buffer), so outputs must agree bit for bit.  Each case
makes two calls in a row through the allocation-free entry point, the second on a smaller batch
(the scratch array keeps the first call's contents), on the T <= 64 decode kernel, the 64 < T <= 256
decode kernel, the prefill path and the float32 path.  Batches that need more scratch than the
array holds are refused before any device work, with y left untouched."""
import numpy as np
import pytest
import torch

import rank_gemm_unified_amd as rg
from gpu_helpers import device_pool, ids_ranks_scale, say
from workloads import custom

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _both(pool, w, T):
    """lora_project and lora_project_noalloc on the first T tokens; returns both outputs."""
    x = w.x()[:T]
    ids = w.ids[:T]
    d_ids, d_ranks, d_scale = ids_ranks_scale(w, ids)
    y_ref = torch.empty_like(x)
    pool.project(0, x, w.W(0), d_ids, d_ranks, d_scale, y=y_ref)
    y = torch.full_like(x, float("nan"))
    rg.lora_project_noalloc(pool.handle, x, w.W(0), pool.table[0], d_ids, d_ranks, d_scale, T, y)
    torch.cuda.synchronize()
    assert rg.lora_check_device_errors(pool.handle, check=False) == 0, rg.lora_last_error()
    return y, y_ref


@pytest.mark.parametrize("H,T1,T2,dtype", [(4096, 64, 17, "bf16"), (4096, 256, 100, "bf16"),
                                           (4096, 1200, 300, "bf16"), (512, 300, 5, "f32")])
def test_noalloc_matches_project(H, T1, T2, dtype):
    rng = np.random.default_rng(T1 + T2)
    ranks = [int(r) for r in rng.choice([8, 16, 32, 64], 24)] + [0]
    ids = rng.integers(-1, 25, T1).astype(np.int32)
    w = custom(H, ranks, ids, dtype=dtype, device="cuda", seed=T1 * 7 + T2)
    say(f"case noalloc H={H} T={T1} then T={T2} {dtype}")
    pool = device_pool(w)
    for T in (T1, T2):
        y, y_ref = _both(pool, w, T)
        assert torch.equal(_bits(y), _bits(y_ref)), T
    pool.close()


def test_noalloc_refuses_oversize_batches():
    w = custom(4096, [16], np.zeros(8, np.int32), device="cuda", seed=3)
    pool = device_pool(w)
    limit = rg.LORA_NOALLOC_SCRATCH_MB << 20
    T = 1 << 16                                   # a prefill batch whose workspace exceeds the limit
    assert rg.lora_project_workspace_size(pool.handle, T) > limit
    d_ids, d_ranks, d_scale = ids_ranks_scale(w)
    x = w.x()
    y = torch.full_like(x, 3.0)
    rc = rg.lora_project_noalloc(pool.handle, x, w.W(0), pool.table[0], d_ids, d_ranks, d_scale, T, y, check=False)
    assert rc == rg.LORA_EINVAL and "scratch" in rg.lora_last_error()
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
    # the largest decode batch at this width fits
    assert rg.lora_project_workspace_size(pool.handle, 256) <= limit
    pool.close()
