"""Pins of the projection oracle against facts that do not come from the oracle itself.

Each pin takes the projection function under test, so the same suite is also run against
deliberately broken copies of it (planted on the CPU, below) to show that a plausible mistake --
a dropped term, a wrong sign, a transposed operand, a wrong adapter or row, a missing scale --
fails at least one pin.
"""
import itertools

import numpy as np
import pytest

import oracle
from oracle import merged_weight, project, project_loops


def _rand_case(seed, T=7, H=12, ranks=(3, 0, 3, 2), with_none=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    W = rng.standard_normal((H, H))
    A = {a: rng.standard_normal((H, r)) for a, r in enumerate(ranks)}
    B = {a: rng.standard_normal((r, H)) for a, r in enumerate(ranks)}
    ids = rng.integers(-1 if with_none else 0, len(ranks), T)
    scale = rng.uniform(0.5, 3.0, len(ranks))
    return x, W, A, B, ids, scale


# ---- pins ------------------------------------------------------------------------------------

def pin_merge_identity(fn):
    """Unmerged == merged: rows of adapter a equal x W' with W' = W + s A B ("Merge or keep
    adapters separate").  Identity rows equal x W."""
    for seed in range(3):
        x, W, A, B, ids, s = _rand_case(seed)
        y = np.asarray(fn(x, W, A, B, ids, s))
        for t in range(x.shape[0]):
            a = int(ids[t])
            Wp = W if a < 0 else merged_weight(W, A[a], B[a], s[a])
            ref = np.array([sum(x[t, k] * Wp[k, n] for k in range(x.shape[1])) for n in range(W.shape[1])])
            if not np.allclose(y[t], ref, rtol=1e-12, atol=1e-12):
                return False
    return True


def pin_closed_form(fn):
    """Integer case with a closed form: W a permutation matrix, A's columns one-hot, B's rows
    c_j times a one-hot.  Then (xW)[n] = x[pi^-1(n)] and the low-rank term adds
    s * c_j * x[k_j] at output m_j.  Computed by indexing, with no products of matrices."""
    H, T = 9, 5
    rng = np.random.default_rng(11)
    pi = rng.permutation(H)                 # W[k, pi[k]] = 1
    W = np.zeros((H, H))
    W[np.arange(H), pi] = 1.0
    inv = np.argsort(pi)
    adapters = {0: ([2, 7, 7], [1, 4, 8], [3, -2, 5], 2.0), 1: ([0], [0], [1], 4.0)}
    A, B, scale = {}, {}, np.zeros(3)
    for a, (ks, ms, cs, s) in adapters.items():
        r = len(ks)
        A[a] = np.zeros((H, r))
        B[a] = np.zeros((r, H))
        for j in range(r):
            A[a][ks[j], j] = 1.0
            B[a][j, ms[j]] = cs[j]
        scale[a] = s
    A[2], B[2] = np.zeros((H, 0)), np.zeros((0, H))        # rank-0 adapter
    x = rng.integers(-4, 5, (T, H)).astype(np.float64)
    ids = np.array([0, 1, -1, 2, 0])
    want = np.zeros((T, H))
    for t in range(T):
        for n in range(H):
            want[t, n] = x[t, inv[n]]
        a = int(ids[t])
        if a in adapters:
            ks, ms, cs, s = adapters[a]
            for k, m, c in zip(ks, ms, cs):
                want[t, m] += s * c * x[t, k]
    return np.array_equal(np.asarray(fn(x, W, A, B, ids, scale)), want)


def pin_brute_force(fn):
    """Agreement with the scalar-loop evaluation of the same definition on tiny inputs."""
    for seed in range(3):
        x, W, A, B, ids, s = _rand_case(100 + seed, T=4, H=6, ranks=(2, 1, 0))
        y = np.asarray(fn(x, W, A, B, ids, s))
        if not np.allclose(y, np.array(project_loops(x, W, A, B, ids, s)), rtol=1e-12, atol=1e-12):
            return False
    return True


def pin_token_permutation(fn):
    """Permuting tokens (with their ids) permutes the rows of y: a token's result depends only on
    its own x and adapter."""
    x, W, A, B, ids, s = _rand_case(7, T=9)
    p = np.random.default_rng(3).permutation(9)
    y = np.asarray(fn(x, W, A, B, ids, s))
    yp = np.asarray(fn(x[p], W, A, B, ids[p], s))
    return np.allclose(yp, y[p], rtol=1e-13, atol=1e-13)


def pin_scale_linear(fn):
    """The low-rank term is linear in its scale: y(2s) - y(0) = 2 (y(s) - y(0))."""
    x, W, A, B, ids, s = _rand_case(5, with_none=False)
    y0 = np.asarray(fn(x, W, A, B, ids, np.zeros_like(s)))
    y1 = np.asarray(fn(x, W, A, B, ids, s))
    y2 = np.asarray(fn(x, W, A, B, ids, 2 * s))
    base = x @ W
    return np.allclose(y2 - y0, 2 * (y1 - y0), rtol=1e-10, atol=1e-10) and np.allclose(y0, base, rtol=1e-12, atol=1e-12)


PINS = [pin_merge_identity, pin_closed_form, pin_brute_force, pin_token_permutation, pin_scale_linear]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    assert pin(project)


def test_loops_pass_closed_form():
    assert pin_closed_form(lambda *a: np.array(project_loops(*a)))


# ---- planted mistakes (CPU only) ---------------------------------------------------------------

def _mutant(kind):
    def fn(x, W, A, B, ids, scale):
        x = np.asarray(x, np.float64)
        Wm = W.T if kind == "transpose_W" else W
        y = x @ Wm
        if kind == "drop_lora":
            return y
        uniq = [int(a) for a in np.unique(ids)]
        for a in uniq:
            if a < 0 or A[a].shape[1] == 0:
                continue
            rows = np.nonzero(ids == a)[0]
            src = rows[::-1] if kind == "wrong_rows" else rows
            b = a
            if kind == "wrong_adapter":
                cands = [c for c in uniq if c >= 0 and c != a and A[c].shape[1] == A[a].shape[1]]
                b = cands[0] if cands else a
            Aa, Ba = A[a], B[b]
            if kind == "drop_index":
                Aa, Ba = Aa[:, 1:], Ba[1:]
            s = float(scale[a])
            if kind == "no_scale":
                s = 1.0
            if kind == "inv_scale":
                s = 1.0 / s if s else 0.0
            term = s * ((x[src] @ Aa) @ Ba)
            y[rows] += -term if kind == "sign" else term
        return y
    return fn


MUTANTS = ["transpose_W", "drop_lora", "wrong_rows", "wrong_adapter", "drop_index", "no_scale",
           "inv_scale", "sign"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    fn = _mutant(kind)
    caught = [p.__name__ for p in PINS if not p(fn)]
    assert caught, f"mutant {kind} passed every pin"


def test_wrong_adapter_mutant_changes_something():
    # the wrong-adapter mutant needs two adapters of equal rank to differ from the oracle
    x, W, A, B, ids, s = _rand_case(1, ranks=(3, 3, 3))
    assert not np.allclose(_mutant("wrong_adapter")(x, W, A, B, ids, s), project(x, W, A, B, ids, s))


# ---- worked and exact small cases -------------------------------------------------------------

def test_identity_adapter_and_none_give_base():
    """Identity (id -1) and a rank-0 adapter both return x W (routing page's "identity" adapter)."""
    x, W, A, B, ids, s = _rand_case(9, ranks=(0, 0))
    ids = np.array([-1, 0, 1, -1, 0, 1, 0])
    y = project(x, W, A, B, ids, s)
    assert np.allclose(y, np.array(project_loops(x, W, {}, {}, ids, s)), rtol=1e-13, atol=1e-13)


def test_integer_case_exact():
    """Entries in {-1, 0, 1}: every partial sum is a small integer, so the fp64 result is exact and
    equals the scalar-loop result bit for bit."""
    rng = np.random.default_rng(5)
    H, T = 16, 6
    x = rng.integers(-1, 2, (T, H)).astype(float)
    W = rng.integers(-1, 2, (H, H)).astype(float)
    A = {0: rng.integers(-1, 2, (H, 4)).astype(float), 1: rng.integers(-1, 2, (H, 2)).astype(float)}
    B = {0: rng.integers(-1, 2, (4, H)).astype(float), 1: rng.integers(-1, 2, (2, H)).astype(float)}
    ids = np.array([0, 1, -1, 1, 0, 0])
    s = np.array([2.0, 1.0])
    y = project(x, W, A, B, ids, s)
    assert np.array_equal(y, np.array(project_loops(x, W, A, B, ids, s)))
    assert np.all(y == np.round(y))


def test_w_identity_special_case():
    """W = I gives y = x + s (x A) B."""
    rng = np.random.default_rng(2)
    H = 8
    x = rng.standard_normal((3, H))
    A = {0: rng.standard_normal((H, 2))}
    B = {0: rng.standard_normal((2, H))}
    y = project(x, np.eye(H), A, B, np.array([0, 0, -1]), np.array([1.5]))
    lo = np.array(project_loops(x[:2], np.zeros((H, H)), A, B, np.array([0, 0]), np.array([1.5])))
    assert np.allclose(y[:2], x[:2] + lo, rtol=1e-13, atol=1e-13)
    assert np.array_equal(y[2], x[2])


@pytest.mark.parametrize("k", [-3, 1, 4])
def test_power_of_two_scaling(k):
    x, W, A, B, ids, s = _rand_case(3)
    y = project(x, W, A, B, ids, s)
    assert np.array_equal(project(x * 2.0 ** k, W, A, B, ids, s), y * 2.0 ** k)


def test_rectangular_shapes_rejected():
    """A and B must be [H][r] and [r][H]: a transposed operand cannot slip through by shape."""
    x, W, A, B, ids, s = _rand_case(4, ranks=(3,), with_none=False)
    with pytest.raises(ValueError):
        project(x, W, {0: A[0].T}, B, ids, s)
    with pytest.raises(ValueError):
        project(x, W, A, {0: B[0].T}, ids, s)


def test_loops_and_numpy_agree_all_small_shapes():
    for T, H, r in itertools.product([1, 3], [2, 5], [1, 2]):
        x, W, A, B, ids, s = _rand_case(T * 31 + H * 7 + r, T=T, H=H, ranks=(r, 0))
        assert np.allclose(project(x, W, A, B, ids, s), np.array(project_loops(x, W, A, B, ids, s)),
                           rtol=1e-12, atol=1e-12)


def test_exports():
    assert callable(oracle.project) and callable(oracle.PagePoolModel)
