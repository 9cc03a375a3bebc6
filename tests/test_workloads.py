"""The seeded generators: determinism, rounding, and the shapes the named workloads promise."""
import time

import numpy as np
import pytest
import torch

from oracle import PagePoolModel
from workloads import build, custom, round_to_bf16


def test_bf16_rounding_matches_rne():
    rng = np.random.default_rng(0)
    a = rng.standard_normal(10000).astype(np.float32)
    # exact ties: low 16 bits = 0x8000, both parities of the kept bit
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40490000], np.uint32).view(np.float32)
    a = np.concatenate([a, ties])
    got = round_to_bf16(a)
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    assert got[-4] == 0x3F80 and got[-3] == 0x3F82      # ties go to even


def test_deterministic():
    a, b = build("tiny"), build("tiny")
    assert np.array_equal(a.ids, b.ids) and np.array_equal(a.free_order, b.free_order)
    assert torch.equal(a.x(), b.x()) and torch.equal(a.W(0), b.W(0))
    assert torch.equal(a.adapter(3)[1], b.adapter(3)[1])
    assert not torch.equal(a.adapter(1)[0], a.adapter(2)[0][:, : a.ranks[1]])


def test_tiny_shape():
    w = build("tiny")
    assert (w.hidden, w.dtype, w.T, w.max_adapters) == (256, "f32", 16, 4)
    assert list(w.ranks) == [4, 8, 8, 16] and list(w.scales) == [4.0, 2.0, 2.0, 1.0]
    At, B = w.adapter(3)
    assert At.shape == (1, 16, 256) and B.shape == (1, 16, 256) and At.dtype == torch.float32
    assert w.ids.min() >= 0 and w.ids.max() < 4


def test_decode_and_prefill_shapes():
    d = build("decode")
    assert (d.hidden, d.T, d.max_adapters, d.dtype) == (4096, 64, 32, "bf16")
    assert set(np.unique(d.ranks)) <= {8, 16, 32, 64}
    p = build("prefill")
    assert p.T == 4096 and list(p.ranks) == [8, 8, 16, 16, 32, 32, 64, 64]
    assert all(np.all(p.ids[s:s + n] == i) for i, (s, n) in enumerate(p.segments))


def test_many_identity_share():
    m = build("many")
    assert m.T == 256 and m.max_adapters == 2001 and m.ranks[2000] == 0
    assert int(np.sum(m.ids == 2000)) == 26
    assert m.slot_x == [0, 0, 0, 1]


def test_stack_rows():
    s = build("stack13b")
    assert s.T == 4 * 2048 + 256 and s.n_slots == 160 and s.hidden == 5120
    for i, (st, n) in enumerate(s.segments):
        assert len(set(s.ids[st:st + n].tolist())) == 1


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "many"])
def test_pool_plans_fit(name):
    w = build(name)
    pool = PagePoolModel(w.num_pages, w.free_order)
    assert all(s == "ok" for s in pool.run(w.ops, w.ranks, w.n_slots))
    st = pool.stats()
    assert 0.5 <= st["kv_pages"] / st["num_pages"] <= 0.61
    assert 0.0 <= st["free_pages"] / st["num_pages"] <= 0.08
    assert st["resident_adapters"] == w.max_adapters


def test_stack_plan_churn_and_fragmentation():
    t0 = time.time()
    w = build("stack13b")
    pool = PagePoolModel(w.num_pages, w.free_order)
    st = pool.run(w.ops, w.ranks, w.n_slots)
    assert all(s == "ok" for s in st)
    assert sum(1 for o in w.ops if o[0] == "evict") > 100
    stats = pool.stats()
    assert 0.10 <= stats["kv_pages"] / stats["num_pages"] <= 0.16
    # consecutive entries of an adapter's table row rarely sit in adjacent physical pages
    adj = tot = 0
    for aid in range(0, w.max_adapters, 37):
        pt = pool.page_table(7, w.max_adapters, 64)[aid]
        r = int(w.ranks[aid])
        row = pt[: 2 * r]
        adj += int(np.sum(np.abs(np.diff(row)) == 1))
        tot += row.size - 1
    assert adj / tot <= 0.10
    assert time.time() - t0 < 120


def test_custom_int_values():
    w = custom(16, [2, 3], [0, 1, -1], values="int")
    x = w.x()
    assert set(torch.unique(x.float()).tolist()) <= {-1.0, 0.0, 1.0}
    assert w.ops and w.num_pages >= 10
