"""3D Hilbert-curve token order for visual grids -- TEST INFRASTRUCTURE ONLY.

[chapterpal] method paragraph and recommendations: for visual inputs, reordering
the tokens along a space-filling Hilbert curve improves token locality and so
block sparsity.  The pages name no curve variant; the reading taken is J. Skilling,
"Programming the Hilbert curve", AIP Conf. Proc. 707 (2004): the n-dimensional
curve on a 2^m cube in "transpose" form, axes (t, y, x).

This side implements the INVERSE map (Hilbert index -> cell), written from the
paper's description: the index's bits are dealt round-robin into n words, a Gray
decode follows, then the reflections/exchanges applied while encoding are undone
from the finest level up.  The GPU library independently implements the FORWARD
map (cell -> index) and sorts; the tests require both to give the same order.

Parity status: the curve variant is a convention, pinned by the curve's own
properties (a bijection that starts at the origin, moves one cell per step on
the full cube, and fills aligned sub-cubes contiguously) and by that agreement.
"""

from __future__ import annotations

import numpy as np


def hilbert_index_to_axes(h: np.ndarray, m: int, n: int = 3) -> np.ndarray:
    """Cells of Hilbert indices ``h`` (array of ints < 2^(n*m)); returns (len, n) coords."""
    h = np.asarray(h, dtype=np.int64)
    # Deal the index bits into n words: word i receives bit n*b + (n-1-i) as bit b.
    X = [np.zeros_like(h) for _ in range(n)]
    for b in range(m):
        for i in range(n):
            X[i] |= ((h >> (n * b + (n - 1 - i))) & 1) << b
    # Gray decode across the words.
    t = X[n - 1] >> 1
    for i in range(n - 1, 0, -1):
        X[i] = X[i] ^ X[i - 1]
    X[0] = X[0] ^ t
    # Undo the per-level reflections and axis exchanges, lowest level first.
    Q = 2
    while Q < (1 << m):
        P = Q - 1
        for i in range(n - 1, -1, -1):
            bit = (X[i] & Q) != 0
            # reflection of the lower bits of word 0
            x0_ref = X[0] ^ P
            # exchange of the lower bits between word 0 and word i
            tt = (X[0] ^ X[i]) & P
            x0_ex = X[0] ^ tt
            xi_ex = X[i] ^ tt
            new0 = np.where(bit, x0_ref, x0_ex)
            newi = np.where(bit, X[i], xi_ex)
            X[0] = new0
            if i != 0:
                X[i] = newi
        Q <<= 1
    return np.stack(X, axis=1)


def cube_order(m: int) -> np.ndarray:
    """All cells of the 2^m cube in Hilbert order, shape (8^m, 3) as (t, y, x)."""
    return hilbert_index_to_axes(np.arange(1 << (3 * m)), m, 3)


def hilbert_cell_order(T: int, H: int, W: int) -> np.ndarray:
    """Token permutation of a T x H x W grid (row-major t, y, x) in Hilbert order.

    The grid is placed at the origin of the smallest 2^m cube that holds it; cells
    are taken in curve order, skipping those outside the grid.  Returns int64
    ``perm`` with perm[p] = row-major index of the p-th cell along the curve.
    """
    m = 0
    while (1 << m) < max(T, H, W, 1):
        m += 1
    cells = cube_order(m)
    inside = (cells[:, 0] < T) & (cells[:, 1] < H) & (cells[:, 2] < W)
    c = cells[inside]
    return c[:, 0] * (H * W) + c[:, 1] * W + c[:, 2]


def cube_bits(T: int, H: int, W: int) -> int:
    m = 0
    while (1 << m) < max(T, H, W, 1):
        m += 1
    return m
