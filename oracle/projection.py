"""The projection itself, in float64.  Test infrastructure only (see the package docstring).

Definition ("S-LoRA, in depth", section "Merge or keep adapters separate"): a LoRA adapter turns
an h-by-h weight W into W + AB, A being h-by-r and B r-by-h; a token with activation x gets
xW + (xA)B.  Unmerged serving keeps W shared and adds the low-rank term per request.

Readings taken where the pages are silent (each is listed in the design notes):
  * a per-adapter float scale s_a multiplies the low-rank term: y = xW + s_a (xA_a) B_a
    (the pages' formula is the case s_a = 1);
  * adapter id -1, or a rank-0 adapter, is the weightless "identity" adapter of the routing page's
    registry: y = xW;
  * W is given here in the formula's layout, W[k, n] with k the input index.
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def project(x, W, A: dict, B: dict, ids, scale) -> np.ndarray:
    """y[t] = x[t] W + s_a (x[t] A_a) B_a with a = ids[t]; identity when a < 0 or rank 0.

    x [T][H], W [H][H] (W[k, n]), A[a] [H][r_a], B[a] [r_a][H], ids [T], scale [n_adapters].
    The base product is one matrix product over all tokens, as the page batches it.  The low-rank
    term is the per-token formula evaluated for the rows that share an adapter.
    """
    x = _f64(x)
    W = _f64(W)
    ids = np.asarray(ids)
    y = x @ W
    for a in np.unique(ids):
        a = int(a)
        if a < 0 or a not in A or _f64(A[a]).shape[1] == 0:
            continue
        rows = np.nonzero(ids == a)[0]
        xa = x[rows] @ _f64(A[a])                   # [n_rows][r]
        y[rows] += float(scale[a]) * (xa @ _f64(B[a]))
    return y


def project_loops(x, W, A: dict, B: dict, ids, scale) -> list:
    """The same definition as plain Python loops over scalars (tiny inputs only)."""
    x = [[float(v) for v in row] for row in _f64(x)]
    W = [[float(v) for v in row] for row in _f64(W)]
    H_in, H_out = len(W), len(W[0])
    y = []
    for t, row in enumerate(x):
        out = [0.0] * H_out
        for n in range(H_out):
            acc = 0.0
            for k in range(H_in):
                acc += row[k] * W[k][n]
            out[n] = acc
        a = int(ids[t])
        if a >= 0 and a in A:
            Aa, Ba = _f64(A[a]), _f64(B[a])
            r = Aa.shape[1]
            v = []
            for j in range(r):
                acc = 0.0
                for k in range(H_in):
                    acc += row[k] * float(Aa[k, j])
                v.append(acc)
            s = float(scale[a])
            for n in range(H_out):
                acc = 0.0
                for j in range(r):
                    acc += v[j] * float(Ba[j, n])
                out[n] += s * acc
        y.append(out)
    return y


def merged_weight(W, A_a, B_a, s: float) -> np.ndarray:
    """W' = W + s A B: the merged weight of one adapter (section "Merge or keep adapters separate")."""
    return _f64(W) + float(s) * (_f64(A_a) @ _f64(B_a))


def gather_page_ids(page_table_slot, ids, ranks, max_rank: int) -> np.ndarray:
    """Pages each token's gather reads, in token order: int64 [T][2*max_rank], -1 where none.

    ``page_table_slot[a]`` lists adapter a's pages for one projection: entries 0..r-1 hold the r
    columns of A, entries r..2r-1 the r rows of B (section "Unified paging": A and B of rank r are r
    H-vectors each, one page per vector).  Tokens without an adapter (id -1) or on a rank-0 adapter read
    nothing.
    """
    pt = np.asarray(page_table_slot)
    ids = np.asarray(ids)
    out = np.full((ids.size, 2 * max_rank), -1, dtype=np.int64)
    for t, a in enumerate(ids):
        a = int(a)
        if a < 0:
            continue
        r = int(ranks[a])
        out[t, : 2 * r] = pt[a, : 2 * r]
    return out


def expected_page_rows(page_table_slot, a: int, rank: int, A_t_slot, B_slot):
    """(page id, vector) pairs that adapter a's pages must hold for one projection.

    Page j < r holds column j of A (row j of A^T); page r + j holds row j of B.
    """
    pt = np.asarray(page_table_slot)
    out = []
    for j in range(rank):
        out.append((int(pt[a, j]), np.asarray(A_t_slot[j])))
    for j in range(rank):
        out.append((int(pt[a, rank + j]), np.asarray(B_slot[j])))
    return out
