"""Independent solvers that pin the CPU oracle (test helpers, fp64, tiny sizes).

None of these reuses the oracle's factorisation, sweep or grid code: each restates a
different but equivalent formulation the pages give.

* ``obs_downdate``: the fixed-order Optimal-Brain-Surgeon form — keep the full
  inverse Hessian, compensate with its row, then eliminate the quantized column by the
  rank-one Schur-complement downdate ("Same Ruler, Smarter Placement: GPTQ", 1.5 and
  1.7 "The setup"; "04 — GPTQ: ...", section 2 on OBS/OBQ).
* ``lazy_blocked``: the lazy batch form of "Same Ruler, Smarter Placement: GPTQ", 1.8:
  inside a block of B columns the updates land at once, the block's scaled errors are
  collected and reach the later columns in one product after the block.
* ``babai``: Babai's nearest-plane algorithm on the lattice whose Gram matrix is the
  damped Hessian ("04 — GPTQ: ...", section 4), with a fixed per-row grid.
* ``rtn``: round-to-nearest on the same grid (what GPTQ reduces to when H is
  diagonal: no off-diagonal coupling, so no compensation).

Grids are written out per row segment here: asymmetric min-max, or symmetric with the
zero at the middle level and the step max|w| / (2^(bits-1) - 1).  ``fixed`` gives, per
row and processing position, a grid decided before the sweep (static groups).
"""

from __future__ import annotations

import numpy as np


def segment_grid(w: np.ndarray, bits: int, sym: bool = False):
    """(step, zero level) of one row segment."""
    maxq = 2 ** bits - 1
    if sym:
        half = 2 ** (bits - 1)
        return max(float(np.max(np.abs(w))) / (half - 1), 1e-8), float(half)
    lo = min(0.0, float(np.min(w)))
    hi = max(0.0, float(np.max(w)))
    s = max((hi - lo) / maxq, 1e-8)
    return s, float(np.rint(-lo / s))


def minmax_grid(w: np.ndarray, maxq: int):
    """Asymmetric (step, zero) for a maxq given directly."""
    return segment_grid(w, int(round(np.log2(maxq + 1))), False)


def _code(x: float, s: float, z: float, maxq: int) -> float:
    return float(min(max(np.rint(x / s) + z, 0.0), maxq))


def static_grids(W: np.ndarray, perm: np.ndarray, bits: int, group: int, sym: bool = False) -> np.ndarray:
    """[rows, d, 2]: the (step, zero) each processing position uses when the groups are
    runs of original columns fitted on W (original order) before the sweep."""
    rows, d = W.shape
    out = np.zeros((rows, d, 2))
    for r in range(rows):
        by_col = {}
        for g0 in range(0, d, group):
            sz = segment_grid(W[r, g0:g0 + group], bits, sym)
            for c in range(g0, min(g0 + group, d)):
                by_col[c] = sz
        for q in range(d):
            out[r, q] = by_col[int(perm[q])]
    return out


def obs_downdate(Wp: np.ndarray, Hp_damped: np.ndarray, bits: int, group: int, sym: bool = False,
                 fixed: np.ndarray | None = None) -> np.ndarray:
    """Codes [rows, d] (processing order) from explicit inverse downdates."""
    maxq = 2 ** bits - 1
    rows, d = Wp.shape
    g = d if group == -1 else group
    codes = np.zeros((rows, d))
    for r in range(rows):
        w = Wp[r].astype(np.float64).copy()
        Hinv = np.linalg.inv(Hp_damped)
        s = z = None
        for q in range(d):
            if fixed is not None:
                s, z = fixed[r, q]
            elif q % g == 0:
                s, z = segment_grid(w[q:q + g], bits, sym)
            c = _code(w[q], s, z, maxq)
            codes[r, q] = c
            e = w[q] - s * (c - z)
            # OBS: the other free weights move along the q-th row of the inverse
            w[q + 1:] -= e / Hinv[q, q] * Hinv[q, q + 1:]
            # eliminate q: Schur complement of the inverse
            Hinv = Hinv - np.outer(Hinv[:, q], Hinv[q, :]) / Hinv[q, q]
    return codes


def lazy_blocked(Wp: np.ndarray, U: np.ndarray, bits: int, group: int, block: int, sym: bool = False) -> np.ndarray:
    """Codes [rows, d] (processing order) of the lazy-batch sweep with block size ``block``.

    Within the block [b, e) each quantized column's scaled error is removed from the
    block's later columns right away; the block's errors E [rows, e - b] are removed
    from all columns after the block in one product E @ U[b:e, e:] once the block is done.
    """
    maxq = 2 ** bits - 1
    rows, d = Wp.shape
    g = d if group == -1 else group
    W = Wp.astype(np.float64).copy()
    codes = np.zeros((rows, d))
    steps = np.zeros((rows, 2))
    for b in range(0, d, block):
        e = min(b + block, d)
        E = np.zeros((rows, e - b))
        for q in range(b, e):
            for r in range(rows):
                if q % g == 0:
                    steps[r] = segment_grid(W[r, q:q + g], bits, sym)
                s, z = steps[r]
                c = _code(W[r, q], s, z, maxq)
                codes[r, q] = c
                E[r, q - b] = (W[r, q] - s * (c - z)) / U[q, q]
            for j in range(q + 1, e):
                W[:, j] -= E[:, q - b] * U[q, j]
        if e < d:
            W[:, e:] -= E @ U[b:e, e:]
    return codes


def babai(Wp: np.ndarray, M: np.ndarray, bits: int) -> np.ndarray:
    """Nearest-plane codes with a fixed min-max grid per row.

    M is any basis matrix with M^T M = damped Hessian (columns = basis directions).
    Gram-Schmidt runs from the last column to the first, so the orthogonalised
    direction of column j is orthogonal to every later column; the nearest plane
    then decides j = 0, 1, ... in turn, subtracting each chosen lattice component.
    """
    maxq = 2 ** bits - 1
    rows, d = Wp.shape
    Bs = M.astype(np.float64).copy()
    star = np.zeros_like(Bs)
    for j in range(d - 1, -1, -1):
        v = Bs[:, j].copy()
        for k in range(j + 1, d):
            v -= (v @ star[:, k]) / (star[:, k] @ star[:, k]) * star[:, k]
        star[:, j] = v
    codes = np.zeros((rows, d))
    for r in range(rows):
        s, z = segment_grid(Wp[r], bits)
        t = M @ Wp[r]
        for j in range(d):
            mu = (t @ star[:, j]) / (star[:, j] @ star[:, j]) / s
            c = float(min(max(np.rint(mu) + z, 0.0), maxq))
            codes[r, j] = c
            t = t - s * (c - z) * M[:, j]
    return codes


def rtn(Wp: np.ndarray, bits: int, group: int, sym: bool = False, fixed: np.ndarray | None = None) -> np.ndarray:
    maxq = 2 ** bits - 1
    rows, d = Wp.shape
    g = d if group == -1 else group
    codes = np.zeros((rows, d))
    for r in range(rows):
        for g0 in range(0, d, g):
            s, z = segment_grid(Wp[r, g0:g0 + g], bits, sym)
            for q in range(g0, min(g0 + g, d)):
                if fixed is not None:
                    s, z = fixed[r, q]
                codes[r, q] = _code(Wp[r, q], s, z, maxq)
    return codes
