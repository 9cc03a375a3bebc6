"""The work the bench divides by: bench.algorithmic() against counts made here, token by token, and
against the committed MFMA counters of the prefill GEMM.

"S-LoRA, in depth", section "Kernels for a batch of mixed ranks": the base product reads W once for
all tokens, low-rank work follows tokens and their ranks, adapter memory follows the distinct
adapters of the batch (each A and B page once)."""
import os
import re

import numpy as np

import bench
from workloads import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
E = 2   # bfloat16


def _by_hand(w, slots):
    """(bytes, flops, A-page bytes) of one step, counted over the tokens one at a time."""
    H, T = w.hidden, len(w.ids)
    seen, r_tokens = set(), 0
    for a in w.ids:
        a = int(a)
        if a >= 0:
            r_tokens += int(w.ranks[a])
            if int(w.ranks[a]) > 0:
                seen.add(a)
    a_pages = sum(int(w.ranks[a]) for a in seen) * H * E      # every A page (or every B page) once
    per_call = H * H * E + 2 * T * H * E + 2 * a_pages + 4 * T
    flops = 2 * T * H * H + 4 * H * r_tokens
    return per_call * slots, flops * slots, a_pages


def test_decode_step_work():
    w = build("decode")
    info = bench.algorithmic(w, w.ids, 1)
    nbytes, flops, a_pages = _by_hand(w, 1)
    assert info["bytes"] == nbytes and info["flops"] == flops
    H, T = w.hidden, len(w.ids)
    # first launch: W, x, the A pages, the ids; second: the B pages and y
    assert info["decode_first_bytes"] == H * H * E + T * H * E + a_pages + 4 * T
    assert info["decode_second_bytes"] == a_pages + T * H * E
    # the seeded draw: 28 distinct adapters, 840 A pages of 8 KiB
    assert info["distinct_adapters"] == 28 and a_pages == 840 * 8192
    assert info["decode_first_bytes"] == 40_960_256 and info["bytes"] == 48_365_824


def test_many_adapter_step_work():
    w = build("many")
    info = bench.algorithmic(w, w.ids, 4)
    nbytes, flops, _ = _by_hand(w, 4)
    assert info["bytes"] == nbytes and info["flops"] == flops
    assert info["distinct_adapters"] == 137


def test_prefill_flops_match_the_mfma_counters():
    """The GEMM's algorithmic flops (2 T H^2 + 2 H sum_t r_t) against the bf16 MFMA work the committed
    counters saw: each MOPS is 512 flops, and the only work beyond the algorithmic is the low-rank
    K-extension of the rank-8 adapters, padded to the MFMA's K of 16."""
    w = build("prefill")
    info = bench.algorithmic(w, w.ids, 1)
    H, T = w.hidden, len(w.ids)
    ranks = np.array([int(w.ranks[a]) for a in w.ids if a >= 0])
    assert info["prefill_second_flops"] == 2 * T * H * H + 2 * H * int(ranks.sum()) == 138_445_586_432
    text = open(os.path.join(ROOT, "profiles", "k_prefill_main_mfma_counters_prefill_8x512_H4096.md")).read()
    mops = int(re.search(r"\| SQ_INSTS_VALU_MFMA_MOPS_BF16 \| ([\d,]+) \|", text).group(1).replace(",", ""))
    padding = 2 * H * int(np.maximum(16 - ranks, 0).sum())
    assert mops * 512 == info["prefill_second_flops"] + padding
