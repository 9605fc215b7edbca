"""Independent solvers that pin the CPU oracle (test helpers, fp64, tiny sizes).

None of these reuses the oracle's factorisation, sweep or grid code: each restates a
different but equivalent formulation the pages give.

* ``obs_downdate``: the fixed-order Optimal-Brain-Surgeon form — keep the full
  inverse Hessian, compensate with its row, then eliminate the quantized column by the
  rank-one Schur-complement downdate ("Same Ruler, Smarter Placement: GPTQ", 1.5 and
  1.7 "The setup"; "04 — GPTQ: ...", section 2 on OBS/OBQ).
* ``babai``: Babai's nearest-plane algorithm on the lattice whose Gram matrix is the
  damped Hessian ("04 — GPTQ: ...", section 4), with a fixed per-row grid.
* ``rtn``: round-to-nearest on the same min-max grid (what GPTQ reduces to when H is
  diagonal: no off-diagonal coupling, so no compensation).
"""

from __future__ import annotations

import numpy as np


def minmax_grid(w: np.ndarray, maxq: int):
    """Scale and zero of one row segment, written out per element."""
    lo = min(0.0, float(np.min(w)))
    hi = max(0.0, float(np.max(w)))
    s = max((hi - lo) / maxq, 1e-8)
    return s, float(np.rint(-lo / s))


def _code(x: float, s: float, z: float, maxq: int) -> float:
    return float(min(max(np.rint(x / s) + z, 0.0), maxq))


def obs_downdate(Wp: np.ndarray, Hp_damped: np.ndarray, bits: int, group: int) -> np.ndarray:
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
            if q % g == 0:
                s, z = minmax_grid(w[q:q + g], maxq)
            c = _code(w[q], s, z, maxq)
            codes[r, q] = c
            e = w[q] - s * (c - z)
            # OBS: the other free weights move along the q-th row of the inverse
            w[q + 1:] -= e / Hinv[q, q] * Hinv[q, q + 1:]
            # eliminate q: Schur complement of the inverse
            Hinv = Hinv - np.outer(Hinv[:, q], Hinv[q, :]) / Hinv[q, q]
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
        s, z = minmax_grid(Wp[r], maxq)
        t = M @ Wp[r]
        for j in range(d):
            mu = (t @ star[:, j]) / (star[:, j] @ star[:, j]) / s
            c = float(min(max(np.rint(mu) + z, 0.0), maxq))
            codes[r, j] = c
            t = t - s * (c - z) * M[:, j]
    return codes


def rtn(Wp: np.ndarray, bits: int, group: int) -> np.ndarray:
    maxq = 2 ** bits - 1
    rows, d = Wp.shape
    g = d if group == -1 else group
    codes = np.zeros((rows, d))
    for r in range(rows):
        for g0 in range(0, d, g):
            s, z = minmax_grid(Wp[r, g0:g0 + g], maxq)
            for q in range(g0, min(g0 + g, d)):
                codes[r, q] = _code(Wp[r, q], s, z, maxq)
    return codes
