"""CPU oracle of the GPTQ layer quantizer (fp64, numpy) — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The product path (the
HIP library and its Python binding) never touches it, and it shares no code, table
or helper with that path: it receives the same seeded input bytes and nothing else.

It is a plain, slow, obviously-correct restatement of what the pages compute, in
float64 throughout; library primitives used as single steps are numpy's matmul and
Cholesky, scipy's triangular solve and BLAS rank-one update.  Sources (web pages,
cited by title and section):

* [SRS]  "Same Ruler, Smarter Placement: GPTQ" — 1.4 (H = 2XX^T), 1.5 (the
  compensating update of one column, Steps 1-3), 1.6 (dampening), 1.7 (the Cholesky
  trick: the rows of the upper factor U carry the conditional updates), 1.9
  (activation ordering), 1.11 (a symmetric grid: scale = max|w| / 7 at 4 bits).
* [ARCH] "GPTQ Architecture, in depth" — "The algorithm in code" (Hessian hook,
  dead inputs, act-order, damping, asymmetric min-max group grid refitted at each
  group start), "Groups, act-order and other knobs" (g_idx, symmetric grids, static
  groups), "Packing, tooling and serving".
* [LIN]  "04 — GPTQ: Hessian-Weighted Rounding, the OBS Lineage, and Why It Still
  Ships" — section 1 (objective ||WX - What X||_F^2), section 8 (bit-level layout).
* [ACT]  "GPTQ > ActOrder: Activation-Based Column Ordering" (descending diagonal).

The sweep is the unblocked column-by-column form of [SRS] 1.5: every column's
scaled error reaches all later columns immediately.  The pages' lazy batches of 128
columns ([SRS] 1.8) only change when those updates land, so the unblocked form is the
plain definition the blocked GPU sweep must reproduce.

Readings where the pages are silent or disagree (all listed with reasons in the
design notes of the repository):

* Rounding is round-half-to-even (numpy ``rint``), as the listing's ``torch.round``,
  and a code is the rounded quotient plus the zero point, clamped
  (clamp(round(w / scale) + zero)); the hand example's "half away from zero" remark
  concerns a test-only grid.
* ``group_size = -1`` means one grid per row, fitted once at the first column on the
  whole (dead-zeroed, permuted) row.
* Symmetric grid: the zero point is the middle level 2^(bits-1) and the scale is
  max|w| / (2^(bits-1) - 1), the grid of [SRS] 1.11 (max|w| / 7 at 4 bits) stored
  with an unsigned code.
* Static groups: the groups are runs of consecutive ORIGINAL columns and each group's
  grid is fitted on the dead-zeroed weights before the sweep; every column is
  quantized on the grid of its original group, whatever its processing position.
* ActOrder sorts by the fp64 Hessian diagonal after the dead-input fix, descending,
  ties broken by ascending original index (a stable sort).
* The damping mean is taken over the diagonal after the dead-input fix.
* H is the unnormalised 2 * sum_t x_t x_t^T (scale-invariant for the codes because
  damping is relative); the running-mean form of the hook differs only by 1/n.

Pins (tests/test_oracle_*.py): brute-force H on tiny integer inputs, closed-form
2x2 factor, Schur-complement downdates, damping bounds, an independent explicit-
inverse OBS solver, an independent Babai nearest-plane solver, an independent
lazy-batch (blocked) sweep, the diagonal-H => round-to-nearest invariant, an exact
rounding tie, H-scale invariance, the page's 4x4 worked example, and the page's
checkpoint byte formula.
"""

from __future__ import annotations

import dataclasses

import numpy as np
from scipy.linalg import solve_triangular
from scipy.linalg.blas import dger

__all__ = [
    "NotSPD", "widen", "ref_accumulate_hessian", "ref_channel_energy", "ref_hessian_entries",
    "ref_column_order", "ref_prepare_hinv", "UniformGrid", "obs_sweep", "GridDecisions",
    "ref_quantize_layer", "ref_dequantize", "ref_layer_loss", "ref_pack_int4", "ref_unpack_int4",
    "ref_w4a16_matmul", "ref_gptq_layer",
]


class NotSPD(Exception):
    """The damped Hessian has no Cholesky factor ([ARCH] "Failure modes")."""


# ----------------------------------------------------------------------------- inputs

def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored inputs to float64 (bf16 or fp16 bit patterns, or fp32)."""
    if dtype == "bf16":
        bits = np.ascontiguousarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.ascontiguousarray(x, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ------------------------------------------------------------------ Hessian ([SRS] 1.4)

def ref_accumulate_hessian(X: np.ndarray, dtype: str, H: np.ndarray | None = None,
                           n_seen: int = 0, rows_per_step: int = 8192):
    """H += 2 * X^T X for token-major X [n, d_in]; returns (H, n_seen + n).

    [SRS] 1.4: each row's loss is a quadratic form in X X^T, so the Hessian is
    2 X X^T (there X is d_in x n; here the tokens are rows, hence X^T X).
    [ARCH] "The algorithm in code" accumulates it per calibration batch; the tokens
    are widened exactly to fp64 a slab at a time and added in token order.
    """
    n, d = X.shape
    if H is None:
        H = np.zeros((d, d), dtype=np.float64)
    for t0 in range(0, n, rows_per_step):
        x = widen(X[t0:t0 + rows_per_step], dtype)
        H += 2.0 * (x.T @ x)
    return H, n_seen + n


def ref_channel_energy(X: np.ndarray, dtype: str, rows_per_step: int = 8192) -> np.ndarray:
    """The diagonal of ref_accumulate_hessian alone: 2 * sum_t x_ti^2 per channel i, in
    fp64 and token order, a slab at a time (no d_in x d_in matrix is formed)."""
    import torch   # plain CPU tensor ops: the same sums, spread over the host cores

    n, d = X.shape
    e = torch.zeros(d, dtype=torch.float64)
    for t0 in range(0, n, rows_per_step):
        slab = np.ascontiguousarray(X[t0:t0 + rows_per_step])
        if dtype in ("bf16", "f16"):
            # exact widening to fp32; a 16-bit value has at most 11 significant bits, so
            # its square is exact in fp32, and the sum runs in fp64
            if dtype == "bf16":
                bits = torch.from_numpy(slab.view(np.int16)).to(torch.int32).bitwise_and(0xFFFF)
                x = torch.bitwise_left_shift(bits, 16).view(torch.float32)
            else:
                x = torch.from_numpy(slab.view(np.float16)).to(torch.float32)
            e += 2.0 * (x * x).sum(dim=0, dtype=torch.float64)
        else:
            x = torch.from_numpy(widen(slab, dtype))
            e += 2.0 * (x * x).sum(dim=0)
    return e.numpy()


def ref_hessian_entries(X: np.ndarray, dtype: str, rows: np.ndarray, cols: np.ndarray,
                        rows_per_step: int = 8192) -> np.ndarray:
    """The block H[rows][:, cols] of ref_accumulate_hessian alone, 2 * X[:, rows]^T X[:, cols]."""
    n = X.shape[0]
    B = np.zeros((len(rows), len(cols)), dtype=np.float64)
    for t0 in range(0, n, rows_per_step):
        xr = widen(X[t0:t0 + rows_per_step][:, rows], dtype)
        xc = widen(X[t0:t0 + rows_per_step][:, cols], dtype)
        B += 2.0 * (xr.T @ xc)
    return B


# ----------------------------------------------- dead inputs, ActOrder, damping, U

def ref_column_order(diag: np.ndarray, act_order: bool = False):
    """Steps 1-2 of ref_prepare_hinv from the Hessian diagonal alone: (perm, dead, diag
    with dead inputs set to 1).  [ARCH] "The algorithm in code" (dead inputs), [ACT] and
    [SRS] 1.9 (descending diagonal; ties keep the original order)."""
    diag = np.array(diag, dtype=np.float64, copy=True)
    dead = diag == 0
    diag[dead] = 1.0
    if act_order:
        perm = np.argsort(-diag, kind="stable")
    else:
        perm = np.arange(diag.shape[0])
    return perm.astype(np.int64), dead, diag


def ref_prepare_hinv(H: np.ndarray, damp: float = 0.01, act_order: bool = False):
    """From H to the upper Cholesky factor U of the damped, permuted H^-1.

    Steps in the pages' order ([ARCH] "The algorithm in code"; [SRS] 1.6, 1.7, 1.9):
    1. inputs never active (zero diagonal) get H_ii = 1 (their W columns are zeroed
       by the quantizer);
    2. ActOrder: columns in descending order of the Hessian diagonal ([ACT], [SRS] 1.9);
    3. H_p = H[perm][:, perm];  lambda = damp * mean(diag H_p);  H_p += lambda * I;
    4. the four-step recipe of [SRS] 1.7: L = chol(H_p); H_p^-1 = L^-T L^-1;
       U = upper Cholesky factor of H_p^-1, so that H_p^-1 = U^T U.
    Raises NotSPD when step 4 finds H_p not positive definite.
    """
    H = np.array(H, dtype=np.float64, copy=True)
    d = H.shape[0]
    perm, dead, diag = ref_column_order(np.diag(H), act_order)
    H[np.diag_indices(d)] = diag
    Hp = H[np.ix_(perm, perm)]
    lam = damp * float(np.mean(np.diag(Hp)))
    Hp[np.diag_indices(d)] += lam
    try:
        L = np.linalg.cholesky(Hp)
    except np.linalg.LinAlgError as exc:
        raise NotSPD(str(exc)) from None
    if not np.all(np.isfinite(L)) or np.any(np.diag(L) <= 0):
        raise NotSPD("non-positive pivot")
    Linv = solve_triangular(L, np.eye(d), lower=True)
    Hinv = Linv.T @ Linv                                  # cholesky_inverse(L)
    try:
        U = np.linalg.cholesky(Hinv).T                   # upper: Hinv = U^T U
    except np.linalg.LinAlgError as exc:
        raise NotSPD(str(exc)) from None
    return dict(U=U, perm=perm, dead=dead, lam=lam, Hp=Hp)


# ----------------------------------------------------------- the quantization grid

@dataclasses.dataclass(frozen=True)
class UniformGrid:
    """A grid of 2^bits equally spaced levels, one per row of a weight segment.

    A weight w is represented by the level ``code`` in [0, maxq] as
    What = scale * (code - zero).

    Asymmetric ([ARCH] "The algorithm in code"): the levels cover the segment's range
    widened to contain 0, [lo, hi] = [min(0, min w), max(0, max w)], so the step is
    (hi - lo) / maxq (never below 1e-8) and the level of 0 is -lo / step rounded.
    Symmetric ([ARCH] "Groups, act-order and other knobs"; the grid of [SRS] 1.11):
    the step is max|w| / (2^(bits-1) - 1) (never below 1e-8) and 0 sits at the fixed
    middle level 2^(bits-1).
    """

    bits: int
    sym: bool = False

    @property
    def maxq(self) -> int:
        return 2 ** self.bits - 1

    def fit(self, seg: np.ndarray):
        """Per row of ``seg`` [rows, k]: (scale, zero, zero before rounding)."""
        if self.sym:
            half = 2 ** (self.bits - 1)
            scale = np.maximum(np.max(np.abs(seg), axis=1) / (half - 1), 1e-8)
            zero = np.full(seg.shape[0], float(half))
            return scale, zero, zero.copy()
        lo = np.minimum(seg.min(axis=1), 0.0)
        hi = np.maximum(seg.max(axis=1), 0.0)
        scale = np.maximum((hi - lo) / self.maxq, 1e-8)
        zero_pre = -lo / scale
        return scale, np.rint(zero_pre), zero_pre

    def code(self, w: np.ndarray, scale: np.ndarray, zero: np.ndarray):
        """(code, value before rounding in level units) of each weight: the quotient
        w / scale is rounded to the nearest integer (ties to even), the zero point is
        added, and the result is clamped to [0, maxq]."""
        quot = w / scale
        return np.clip(np.rint(quot) + zero, 0, self.maxq), quot + zero


# -------------------------------------------- column sweep ([SRS] 1.5 and 1.7, unblocked)

def obs_sweep(Wp: np.ndarray, U: np.ndarray, quantize_column) -> np.ndarray:
    """GPTQ over the columns of Wp [rows, cols] in order; Wp is modified in place.

    For column q ([SRS] 1.5, Steps 1-3, with the conditional inverse read off the rows of
    the upper factor U, [SRS] 1.7): the current column becomes What_q =
    ``quantize_column(q, Wp)``; its error scaled by the conditional inverse diagonal,
    delta_q = (Wp_q - What_q) / U_qq, is taken out of every later column at once,
    Wp[:, j] -= delta_q * U[q, j] for j > q.  The rank-one update is one BLAS call on a
    column-major copy.  Returns What [rows, cols].
    """
    rows, cols = Wp.shape
    Wf = np.asfortranarray(Wp, dtype=np.float64)
    What = np.zeros((rows, cols))
    for q in range(cols):
        What[:, q] = quantize_column(q, Wf)
        delta = (Wf[:, q] - What[:, q]) / U[q, q]
        if q + 1 < cols:
            later = Wf[:, q + 1:]
            out = dger(-1.0, delta, np.ascontiguousarray(U[q, q + 1:]), a=later, overwrite_a=1)
            if not np.shares_memory(out, later):   # BLAS had to copy: write it back
                later[...] = out
    Wp[...] = Wf
    return What


@dataclasses.dataclass
class GridDecisions:
    """The grid decisions of one sweep ([ARCH] "The algorithm in code" and "Groups,
    act-order and other knobs"), as the per-column callback of :func:`obs_sweep`.

    Per-row (group_size = -1): one grid per row, fitted at column 0 on the whole row.
    Groups: the grid of the group of g consecutive processing positions is refitted on
    the current (already compensated) weights at the group's first position.  Static
    groups: ``static_fit`` holds (scale, zero, zero before rounding) of every group of
    g consecutive ORIGINAL columns, fitted before the sweep; processing position q uses
    the grid of group perm[q] // g.

    With ``forced_codes`` / ``forced_zeros`` (processing order; zeros per stored group)
    the integer decisions are taken from the caller instead (teacher-forced replay);
    every place where a forced integer differs from this oracle's own rounding is
    recorded with the distance of the oracle's value before rounding from the midpoint
    between the two integers.
    """

    rows: int
    cols: int
    grid: UniformGrid
    group_size: int
    perm: np.ndarray | None = None
    static_fit: tuple | None = None
    forced_codes: np.ndarray | None = None
    forced_zeros: np.ndarray | None = None

    def __post_init__(self):
        self.g = self.cols if self.group_size == -1 else self.group_size
        self.n_groups = -(-self.cols // self.g)
        self.codes = np.zeros((self.rows, self.cols), dtype=np.int64)
        self.pre = np.zeros((self.rows, self.cols))           # w/scale + zero
        self.scales = np.zeros((self.n_groups, self.rows))
        self.zeros = np.zeros((self.n_groups, self.rows), dtype=np.int64)
        self.zero_pre = np.zeros((self.n_groups, self.rows))
        self.code_div = []     # (row, col, |v - midpoint|, |code_a - code_b|)
        self.zero_div = []     # (group, row, |v - midpoint|, |zero_a - zero_b|)
        self._cur = None
        if self.static_fit is not None:
            for gi in range(self.n_groups):
                s, z, zp = (np.asarray(a[gi], dtype=np.float64) for a in self.static_fit)
                self._set_group(gi, s, z, zp)

    @staticmethod
    def _gap(v, a, b):
        return np.abs(v - 0.5 * (a + b)), np.abs(a - b)

    def _set_group(self, gi, scale, zero, zero_pre):
        if self.forced_zeros is not None and not self.grid.sym:
            fz = self.forced_zeros[gi].astype(np.float64)
            bad = np.nonzero(fz != zero)[0]
            gap, dist = self._gap(zero_pre[bad], zero[bad], fz[bad])
            self.zero_div += [(gi, int(r), float(g_), float(d_)) for r, g_, d_ in zip(bad, gap, dist)]
            zero = fz
        self.scales[gi], self.zeros[gi], self.zero_pre[gi] = scale, zero, zero_pre

    def __call__(self, q: int, Wf: np.ndarray) -> np.ndarray:
        if self.static_fit is not None:
            gi = int(self.perm[q]) // self.g
        else:
            gi = q // self.g
            if q % self.g == 0:
                self._set_group(gi, *self.grid.fit(Wf[:, q:q + self.g]))
        scale, zero = self.scales[gi], self.zeros[gi].astype(np.float64)
        code, v = self.grid.code(Wf[:, q], scale, zero)
        if self.forced_codes is not None:
            fc = self.forced_codes[:, q].astype(np.float64)
            bad = np.nonzero(fc != code)[0]
            gap, dist = self._gap(v[bad], code[bad], fc[bad])
            self.code_div += [(int(r), q, float(g_), float(d_)) for r, g_, d_ in zip(bad, gap, dist)]
            code = fc
        self.pre[:, q] = v
        self.codes[:, q] = code
        return scale * (code - zero)


def ref_quantize_layer(W: np.ndarray, dtype: str, prep: dict, bits: int = 4,
                       group_size: int = 128, sym: bool = False, static_groups: bool = False,
                       forced_codes: np.ndarray | None = None,
                       forced_zeros: np.ndarray | None = None):
    """GPTQ of one layer given the output of :func:`ref_prepare_hinv`.

    W [d_out, d_in] (stored dtype) -> codes [d_out, d_in] in ORIGINAL column order,
    scales / zeros [n_groups, d_out], g_idx [d_in] (group of each original column,
    [ARCH] "Groups, act-order and other knobs"), perm, and the dequantized What in
    original order.  Groups are runs of processing positions, or of original columns
    with ``static_groups`` (fitted before the sweep on the dead-zeroed W).
    ``forced_codes`` (original order) / ``forced_zeros`` switch on the replay.
    """
    U, perm, dead = prep["U"], prep["perm"], prep["dead"]
    Wf = widen(W, dtype)
    rows, cols = Wf.shape
    Wf[:, dead] = 0.0
    grid = UniformGrid(bits, sym)
    static = static_groups and group_size != -1
    static_fit = None
    if static:
        fits = [grid.fit(Wf[:, c:c + group_size]) for c in range(0, cols, group_size)]
        static_fit = tuple(np.array([f[i] for f in fits]) for i in range(3))
    Wp = Wf[:, perm].copy()
    fc = None if forced_codes is None else np.asarray(forced_codes)[:, perm]
    dec = GridDecisions(rows, cols, grid, group_size, perm=perm, static_fit=static_fit, forced_codes=fc,
                        forced_zeros=forced_zeros)
    What_p = obs_sweep(Wp, U, dec)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(cols)
    codes = dec.codes[:, inv].astype(np.uint8)
    if static:
        g_idx = (np.arange(cols) // group_size).astype(np.int32)
    else:
        g_idx = (inv // dec.g).astype(np.int32)
    return dict(codes=codes, scales=dec.scales, zeros=dec.zeros.astype(np.uint8),
                g_idx=g_idx, perm=perm, What=What_p[:, inv], grid=dec)


def ref_dequantize(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                   g_idx: np.ndarray) -> np.ndarray:
    """What[o, c] = scale[g_idx[c], o] * (code[o, c] - zero[g_idx[c], o]) in fp64."""
    s = np.asarray(scales, dtype=np.float64)[g_idx].T
    z = np.asarray(zeros, dtype=np.float64)[g_idx].T
    return s * (codes.astype(np.float64) - z)


# ------------------------------------------------------------- objective ([LIN] §1)

def ref_layer_loss(W: np.ndarray, dtype: str, What: np.ndarray, H: np.ndarray) -> float:
    """||W X - What X||_F^2 = 1/2 tr(D H D^T), D = W - What, H = 2 X X^T undamped."""
    D = widen(W, dtype) - What
    return 0.5 * float(np.einsum("ij,ij->", D @ H, D))


# ------------------------------------------------- checkpoint layout ([LIN] §8, [ARCH])

def ref_pack_int4(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray):
    """Eight 4-bit values per int32, element k in bits [4k, 4k+4).

    qweight [d_in/8, d_out] packs codes along the input dimension; qzeros
    [n_groups, d_out/8] packs zero points along the output dimension; scales become
    fp16 (round to nearest even) [n_groups, d_out].
    """
    codes = np.asarray(codes, dtype=np.uint32)
    d_out, d_in = codes.shape
    ct = codes.T.reshape(d_in // 8, 8, d_out)
    qweight = np.zeros((d_in // 8, d_out), dtype=np.uint32)
    for k in range(8):
        qweight |= ct[:, k, :] << np.uint32(4 * k)
    z = np.asarray(zeros, dtype=np.uint32)
    ng = z.shape[0]
    zt = z.reshape(ng, d_out // 8, 8)
    qzeros = np.zeros((ng, d_out // 8), dtype=np.uint32)
    for k in range(8):
        qzeros |= zt[:, :, k] << np.uint32(4 * k)
    return (qweight.view(np.int32), qzeros.view(np.int32),
            np.asarray(scales, dtype=np.float64).astype(np.float16))


def ref_unpack_int4(qweight: np.ndarray, qzeros: np.ndarray):
    """Inverse of the nibble packing: codes [d_out, d_in] and zeros [n_groups, d_out]."""
    qw = np.asarray(qweight).view(np.uint32)
    rows8, d_out = qw.shape
    codes = np.zeros((rows8 * 8, d_out), dtype=np.uint8)
    for k in range(8):
        codes[k::8] = (qw >> np.uint32(4 * k)) & np.uint32(15)
    qz = np.asarray(qzeros).view(np.uint32)
    ng, c8 = qz.shape
    zeros = np.zeros((ng, c8 * 8), dtype=np.uint8)
    for k in range(8):
        zeros[:, k::8] = (qz >> np.uint32(4 * k)) & np.uint32(15)
    return codes.T.copy(), zeros


# ------------------------------------- serving: W4A16 product from the checkpoint tensors

def ref_w4a16_matmul(X: np.ndarray, dtype: str, qweight: np.ndarray, qzeros: np.ndarray,
                     scales_f16: np.ndarray, g_idx: np.ndarray) -> np.ndarray:
    """Y = X What^T in fp64 from the packed checkpoint ([ARCH] "Packing, tooling and serving":
    4-bit weights with 16-bit activations, dequantized right before the product; [LIN]
    section 8 for the tensors).  X [m, d_in] (bf16 / fp16 bits, or fp32); the weights are
    unpacked, each dequantized with its fp16 scale and zero of group g_idx[c], and the
    product is taken in fp64.  Returns Y [m, d_out]."""
    codes, zeros = ref_unpack_int4(qweight, qzeros)
    scales = np.asarray(scales_f16, dtype=np.float16).astype(np.float64)
    What = ref_dequantize(codes, scales, zeros, np.asarray(g_idx))
    return widen(X, dtype) @ What.T


# ------------------------------------------------------------------- whole layer

def ref_gptq_layer(W: np.ndarray, X_chunks, dtype: str, bits: int = 4, group_size: int = 128,
                   damp: float = 0.01, act_order: bool = False, sym: bool = False,
                   static_groups: bool = False, timings: dict | None = None):
    """Hessian -> prepare -> quantize for one layer; ``X_chunks`` is an iterable of
    token-major activation slabs.  Per-stage wall times go to ``timings``."""
    import time
    t0 = time.perf_counter()
    H, n = None, 0
    for Xc in X_chunks:
        H, n = ref_accumulate_hessian(Xc, dtype, H, n)
    if H is None:
        H = np.zeros((W.shape[1], W.shape[1]))
    t1 = time.perf_counter()
    prep = ref_prepare_hinv(H, damp, act_order)
    t2 = time.perf_counter()
    res = ref_quantize_layer(W, dtype, prep, bits, group_size, sym, static_groups)
    t3 = time.perf_counter()
    if timings is not None:
        timings.update(hessian=t1 - t0, prepare=t2 - t1, quantize=t3 - t2)
    res.update(H=H, n_seen=n, prep=prep)
    return res
