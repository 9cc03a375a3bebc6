"""GPU parity of the prefill-shaped path (T > 256: grouped MFMA shrink + tiled MFMA GEMM with the
expand as extra K) against the fp64 oracle, with integer bit-exact cases and bitwise invariants."""
import numpy as np
import pytest
import torch

import rank_gemm_unified_amd as rg
from gpu_helpers import bf16_round_f64, device_pool, errors, oracle_y, run, say
from workloads import build, custom, storage_to_f64

pytestmark = pytest.mark.gpu

BF16_REL, BF16_ABS = 1e-2, 5e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def prefill():
    w = build("prefill", device="cuda")
    say("case prefill: H", w.hidden, "T", w.T)
    pool = device_pool(w)
    y = run(pool, w, 0)
    torch.cuda.synchronize()
    return w, pool, y


def test_prefill_parity(prefill):
    w, pool, y = prefill
    assert rg.lora_check_device_errors(pool.handle, check=False) == 0, rg.lora_last_error()
    ref = oracle_y(w, 0)
    rel, mx = errors(y, ref)
    say(f"prefill relL2={rel:.3e} maxabs={mx:.3e}")
    assert rel <= BF16_REL and mx <= BF16_ABS
    # per-token low-rank delta against the oracle's, on every token
    y0 = run(pool, w, 0, ids=np.full(w.T, -1, np.int32))
    base = oracle_y(w, 0, ids=np.full(w.T, -1, np.int32))
    d_gpu = storage_to_f64(y) - storage_to_f64(y0)
    d_ref = ref - base
    rel_t = np.linalg.norm(d_gpu - d_ref, axis=1) / np.linalg.norm(d_ref, axis=1)
    assert rel_t.max() <= 0.1, (int(rel_t.argmax()), float(rel_t.max()))


def test_prefill_token_permutation_bitwise(prefill):
    """A token's result depends only on its own x and adapter: permuting the tokens permutes the
    rows of y bit for bit."""
    w, pool, y = prefill
    perm = np.random.default_rng(0).permutation(w.T)
    yp = run(pool, w, 0, ids=w.ids[perm], x=w.x()[torch.as_tensor(perm, device="cuda")])
    torch.cuda.synchronize()
    assert torch.equal(yp.view(torch.int16), y[torch.as_tensor(perm, device="cuda")].view(torch.int16))


def test_prefill_identity_and_scaling_bitwise(prefill):
    w, pool, y = prefill
    ids = w.ids.copy()
    ids[1000:1700] = -1                   # part of a segment and a tile boundary
    yi = run(pool, w, 0, ids=ids)
    y0 = run(pool, w, 0, ids=np.full(w.T, -1, np.int32))
    y2 = run(pool, w, 0, x=w.x() * 2)
    torch.cuda.synchronize()
    sel = torch.as_tensor(ids == -1, device="cuda")
    assert torch.equal(yi[sel].view(torch.int16), y0[sel].view(torch.int16))
    assert torch.equal(yi[~sel].view(torch.int16), y[~sel].view(torch.int16))
    assert torch.equal((y.float() * 2).to(torch.bfloat16).view(torch.int16), y2.view(torch.int16))


def _segments(rng, T, n_ad, pieces):
    cuts = np.sort(rng.choice(np.arange(1, T), pieces - 1, replace=False))
    bounds = np.concatenate([[0], cuts, [T]])
    ids = np.empty(T, np.int32)
    for i in range(pieces):
        ids[bounds[i]:bounds[i + 1]] = rng.integers(-1, n_ad)
    return ids


@pytest.mark.parametrize("T,H,pieces", [(257, 64, 3), (300, 128, 7), (549, 192, 5), (1000, 256, 40),
                                        (777, 256, 777)])
def test_prefill_integer_exact(T, H, pieces):
    """Integer inputs keep every partial sum exact (|v| <= H <= 256 is exact in bfloat16), so the
    output must equal the oracle's exact result rounded once to bfloat16.  Segments are ragged,
    tiles straddle segments, the last tile is partial, and pieces == T makes every row its own run."""
    rng = np.random.default_rng(T + H)
    ranks = [4, 1, 0, 16, 2, 64, 33]
    ids = _segments(rng, T, len(ranks), pieces)
    w = custom(H, ranks, ids, values="int", scales=[1] * len(ranks), device="cuda", seed=T)
    say("case prefill int-exact", T, H, pieces)
    pool = device_pool(w)
    y = run(pool, w, 0)
    torch.cuda.synchronize()
    assert rg.lora_check_device_errors(pool.handle, check=False) == 0, rg.lora_last_error()
    ref = oracle_y(w, 0)
    assert np.all(ref == np.round(ref))
    got = y.cpu().view(torch.int16)
    want = bf16_round_f64(ref).view(torch.int16)
    bad = (got != want).any(dim=1).nonzero().flatten().tolist()
    assert not bad, (bad[:10], ids[bad[:10]])


def test_prefill_many_adapters_integer_exact():
    """2000 tokens over 300 adapters (some tokens with none): about 330 shrink work items, so each
    workgroup of the persistent shrink grid takes several (item, split) units and stops at the first
    record past the last item.  Integer inputs: the output must equal the oracle's exact result
    rounded once to bfloat16, on every row."""
    T, H, n_ad = 2000, 256, 300
    rng = np.random.default_rng(2000)
    ranks = [[4, 1, 0, 16, 2, 64, 33, 8][i % 8] for i in range(n_ad)]
    ids = rng.integers(-1, n_ad, T).astype(np.int32)
    w = custom(H, ranks, ids, values="int", scales=[1] * n_ad, device="cuda", seed=T)
    say("case prefill int-exact many adapters", T, H, n_ad)
    pool = device_pool(w)
    y = run(pool, w, 0)
    torch.cuda.synchronize()
    assert rg.lora_check_device_errors(pool.handle, check=False) == 0, rg.lora_last_error()
    ref = oracle_y(w, 0)
    assert np.all(ref == np.round(ref))
    got = y.cpu().view(torch.int16)
    want = bf16_round_f64(ref).view(torch.int16)
    bad = (got != want).any(dim=1).nonzero().flatten().tolist()
    assert not bad, (bad[:10], ids[bad[:10]])


@pytest.mark.parametrize("T,H", [(700, 192), (300, 64)])
def test_prefill_small_max_rank_integer_exact(T, H):
    """A pool whose largest rank is 16: v rows hold 16 entries, so the low-rank operand loads clamp
    inside the row and everything past each adapter's rank (1, 4, 9, 16) is cleared.  Tiles straddle
    several adapters; H = 64 is a single K step."""
    rng = np.random.default_rng(T * 7 + H)
    ranks = [4, 1, 0, 16, 9]
    ids = _segments(rng, T, len(ranks), 30)
    w = custom(H, ranks, ids, values="int", scales=[1] * len(ranks), device="cuda", seed=T + 1)
    w.max_rank = 16
    say("case prefill max_rank 16", T, H)
    pool = device_pool(w)
    y = run(pool, w, 0)
    torch.cuda.synchronize()
    assert rg.lora_check_device_errors(pool.handle, check=False) == 0, rg.lora_last_error()
    ref = oracle_y(w, 0)
    assert np.all(ref == np.round(ref))
    got = y.cpu().view(torch.int16)
    want = bf16_round_f64(ref).view(torch.int16)
    bad = (got != want).any(dim=1).nonzero().flatten().tolist()
    assert not bad, (bad[:10], ids[bad[:10]])


@pytest.mark.parametrize("H", [320, 448, 5120])
def test_prefill_odd_hidden(H):
    """Hidden sizes that are not a multiple of the 256-column tile, with a mixed batch: prefill
    segments and single decode-style rows."""
    rng = np.random.default_rng(H)
    ranks = [8, 16, 32, 64, 0]
    T = 600 if H < 1000 else 520
    ids = np.concatenate([np.full(300, 1), np.full(T - 300 - 60, 3), rng.integers(-1, 5, 60)]).astype(np.int32)
    w = custom(H, ranks, ids, device="cuda", seed=H)
    say("case prefill hidden", H, "T", T)
    pool = device_pool(w)
    y = run(pool, w, 0)
    torch.cuda.synchronize()
    rel, mx = errors(y, oracle_y(w, 0))
    say(f"H={H} relL2={rel:.3e} maxabs={mx:.3e}")
    assert rel <= BF16_REL and mx <= BF16_ABS


def test_prefill_matches_decode_path_within_tolerance():
    """The same 64 tokens through the decode path (T = 64) and embedded in a prefill batch
    (T = 320) agree within the parity bars."""
    rng = np.random.default_rng(9)
    ranks = [8, 16, 64]
    ids = rng.integers(-1, 3, 320).astype(np.int32)
    w = custom(1024, ranks, ids, device="cuda", seed=9)
    pool = device_pool(w)
    y_big = run(pool, w, 0)
    x_small = w.x()[:64].contiguous()
    y_small = run(pool, w, 0, ids=ids[:64], x=x_small)
    torch.cuda.synchronize()
    rel, mx = errors(y_small, storage_to_f64(y_big[:64]))
    assert rel <= BF16_REL and mx <= BF16_ABS


def test_prefill_device_checks_flag_bad_tokens(prefill):
    """The grouping kernel's checks on the prefill path: an out-of-range id, an adapter whose rank
    does not match its page-table row and an adapter whose rank exceeds the pool's are reported in
    the error word; their tokens get the base product bit for bit, every other token is unchanged."""
    w, pool, y_ok = prefill
    assert rg.lora_check_device_errors(pool.handle, check=False) == 0
    ids, ranks = w.ids.copy(), w.ranks.copy()
    ids[5] = 5000                                   # out of range
    a_tab, a_rk = int(ids[600]), int(ids[1200])     # adapters of requests 1 and 2
    assert a_tab != a_rk and min(a_tab, a_rk) >= 0
    ranks[a_tab] = max(int(ranks[a_tab]) // 2, 1)   # not the loaded rank
    ranks[a_rk] = w.max_rank + 5                    # beyond the pool's largest rank
    y = torch.empty_like(w.x())
    rg.lora_project(pool.handle, w.x(), w.W(0), pool.table[0], torch.as_tensor(ids, device="cuda"),
                    torch.as_tensor(ranks, device="cuda"), torch.as_tensor(w.scales, device="cuda"), w.T, y,
                    pool.workspace(w.T))
    assert rg.lora_check_device_errors(pool.handle, check=False) == rg.LORA_EDEVICE
    msg = rg.lora_last_error()
    for part in ("adapter-id-out-of-range", "rank-out-of-range", "adapter-not-loaded-at-this-rank"):
        assert part in msg, msg
    assert rg.lora_check_device_errors(pool.handle, check=False) == 0     # cleared
    bad = (ids == 5000) | (ids == a_tab) | (ids == a_rk)
    y0 = run(pool, w, 0, ids=np.full(w.T, -1, np.int32))
    torch.cuda.synchronize()
    b = torch.as_tensor(bad, device="cuda")
    assert torch.equal(y[b].view(torch.int16), y0[b].view(torch.int16))
    assert torch.equal(y[~b].view(torch.int16), y_ok[~b].view(torch.int16))
