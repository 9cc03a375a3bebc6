"""fp64 CPU oracle for the unmerged multi-LoRA projection and its unified page pool.

TEST INFRASTRUCTURE ONLY.  Nothing in the library calls, imports or links this package; only the
tests, the smoke check and the benchmark's CPU-baseline leg may use it.  It shares no code with the
HIP path: it never imports ``rank_gemm_unified_amd`` and reads inputs only from ``workloads`` (or
from arrays a test hands it).

Sources (the pages this follows):
  * "S-LoRA, in depth" (aicassindra.com), section "Merge or keep adapters separate": the layer
    output for activation x is xW + (xA)B; merging gives W' = W + AB; unmerged serving batches xW
    over every request whatever its adapter.
  * same page, section "The architecture": a gather step fetches each request's A and B pages
    from whatever places in memory hold them.
  * same page, section "Unified paging: adapters and KV cache in one pool" (with its worked
    example and its pool sketch): one page = one H-vector; a rank-R LoRA tensor takes R pages;
    KV and adapters share one free list.
  * "Switch Adapters by Routing Requests Through Resident, Verified State" (tuckerl.ee), the
    adapter registry: requests that name no adapter get an "identity" adapter with no weights;
    an unknown adapter is an error.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against closed forms, the
worked example's printed values (``tests/golden/``), hand-derived traces and brute force.  No
function is parity-unpinned.
"""
from .projection import (  # noqa: F401
    expected_page_rows,
    gather_page_ids,
    merged_weight,
    project,
    project_loops,
)
from .pool import (  # noqa: F401
    PagePoolModel,
    Resident,
    adapter_bytes,
    adapter_page_count,
    h2d_seconds,
    kv_bytes_per_token,
    kv_pages_per_token,
    tp_comm_lora,
    tp_comm_base,
)
