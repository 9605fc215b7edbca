"""CPU oracle of the GPTQ layer quantizer (fp64, numpy) — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The product path (the
HIP library and its Python binding) never touches it, and it shares no code, table
or helper with that path: it receives the same seeded input bytes and nothing else.

It is a plain, slow, obviously-correct restatement of what the pages compute, in
float64 throughout; library primitives used as single steps are numpy's matmul and
Cholesky and scipy's triangular solve.  Sources (web pages, cited by title and
section):

* [SRS]  "Same Ruler, Smarter Placement: GPTQ" — 1.4 (H = 2XX^T), 1.5 (the
  compensating update, Steps 1-3), 1.6 (dampening), 1.7 (the Cholesky trick and its
  four-step recipe), 1.8 (lazy batch update), 1.9 (activation ordering).
* [ARCH] "GPTQ Architecture, in depth" — "The algorithm in code" (Hessian hook,
  min-max group fit, the blocked column loop, dead inputs, act-order, damping),
  "Groups, act-order and other knobs" (g_idx), "Packing, tooling and serving".
* [LIN]  "04 — GPTQ: Hessian-Weighted Rounding, the OBS Lineage, and Why It Still
  Ships" — section 1 (objective ||WX - What X||_F^2), section 8 (bit-level layout).
* [ACT]  "GPTQ > ActOrder: Activation-Based Column Ordering" (descending diagonal).

Readings where the pages are silent or disagree (all listed with reasons in the
design notes of the repository):

* Rounding is round-half-to-even (numpy ``rint``), as the listing's ``torch.round``;
  the hand example's "half away from zero" remark concerns a test-only grid.
* ``group_size = -1`` means one grid per row, fitted once at the first column on the
  whole (dead-zeroed, permuted) row.
* ActOrder sorts by the fp64 Hessian diagonal after the dead-input fix, descending,
  ties broken by ascending original index (a stable sort).
* The damping mean is taken over the diagonal after the dead-input fix.
* H is the unnormalised 2 * sum_t x_t x_t^T (scale-invariant for the codes because
  damping is relative); the running-mean form of the hook differs only by 1/n.

Pins (tests/test_oracle_*.py): brute-force H on tiny integer inputs, closed-form
2x2 factor, Schur-complement downdates, damping bounds, an independent explicit-
inverse OBS solver, an independent Babai nearest-plane solver, the diagonal-H =>
round-to-nearest invariant, block-size and H-scale invariance, the page's 4x4
worked example, and the page's checkpoint byte formula.
"""

from __future__ import annotations

import dataclasses

import numpy as np
from scipy.linalg import solve_triangular

__all__ = [
    "NotSPD", "widen", "ref_accumulate_hessian", "ref_channel_energy", "ref_hessian_entries",
    "ref_column_order", "ref_prepare_hinv", "fit_minmax",
    "gptq_sweep", "MinMaxGrid", "ref_quantize_layer", "ref_dequantize",
    "ref_layer_loss", "ref_pack_int4", "ref_unpack_int4", "ref_gptq_layer",
]


class NotSPD(Exception):
    """The damped Hessian has no Cholesky factor ([ARCH] "Failure modes")."""


# ----------------------------------------------------------------------------- inputs

def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored inputs to float64 (bf16 bit patterns or fp32)."""
    if dtype == "bf16":
        bits = np.ascontiguousarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
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
        if dtype == "bf16":
            # exact widening of the bf16 bits to fp32; a bf16 value has 8 significant bits,
            # so its square is exact in fp32, and the sum runs in fp64
            bits = torch.from_numpy(slab.view(np.int16)).to(torch.int32).bitwise_and(0xFFFF)
            x = torch.bitwise_left_shift(bits, 16).view(torch.float32)
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


# --------------------------------------------------------------- grid ([ARCH] fit_group)

def fit_minmax(Wg: np.ndarray, maxq: int):
    """Asymmetric min-max grid of each row of Wg: (scale, zero) per row.

    The range always contains 0: lo = min(0, min row), hi = max(0, max row);
    scale = max((hi - lo) / maxq, 1e-8); zero = round(-lo / scale).
    Returns also the pre-rounding zero value -lo/scale (for the replay check).
    """
    lo = np.minimum(Wg.min(axis=1), 0.0)
    hi = np.maximum(Wg.max(axis=1), 0.0)
    scale = np.maximum((hi - lo) / maxq, 1e-8)
    zval = -lo / scale
    return scale, np.rint(zval), zval


# -------------------------------------------------- column sweep ([SRS] 1.5, 1.7, 1.8)

def gptq_sweep(Wp: np.ndarray, U: np.ndarray, block: int, quantize_column) -> np.ndarray:
    """Blocked GPTQ sweep over the columns of Wp (modified in place).

    For each column q in order: the grid turns the current column into What_q
    (``quantize_column(q, Wp)``); err_q = (W_q - What_q) / U_qq; the columns after q
    inside the current block absorb err_q * U[q, q+1:] at once ([SRS] 1.5 Step 3 with
    the rows of U from 1.7); the errors of a finished block are applied to every
    later column in one product Err @ U[block, later] ([SRS] 1.8 lazy batch update,
    which only changes when updates land, not which).  Returns What [rows, cols].
    """
    rows, cols = Wp.shape
    What = np.zeros_like(Wp)
    for i in range(0, cols, block):
        j2 = min(i + block, cols)
        Err = np.zeros((rows, j2 - i))
        for q in range(i, j2):
            What[:, q] = quantize_column(q, Wp)
            err = (Wp[:, q] - What[:, q]) / U[q, q]
            Wp[:, q + 1:j2] -= np.outer(err, U[q, q + 1:j2])
            Err[:, q - i] = err
        if j2 < cols:
            Wp[:, j2:] -= Err @ U[i:j2, j2:]
    return What


@dataclasses.dataclass
class MinMaxGrid:
    """Per-row (group_size=-1) or per-group asymmetric grid of [ARCH] "The algorithm
    in code": at the first column of every group the grid is refitted on the current
    (already compensated) weights of that group; codes are
    q = clamp(round(w / scale) + zero, 0, 2^bits - 1) and What = scale * (q - zero).

    With ``forced_codes`` / ``forced_zeros`` (permuted column order) the decisions are
    taken from the caller instead (teacher-forced replay); every place where the
    forced integer differs from this oracle's own rounding is recorded together with
    the distance of the oracle's pre-rounding value from the midpoint between the
    two integers.
    """

    rows: int
    cols: int
    bits: int
    group_size: int
    forced_codes: np.ndarray | None = None
    forced_zeros: np.ndarray | None = None

    def __post_init__(self):
        self.maxq = 2 ** self.bits - 1
        self.g = self.cols if self.group_size == -1 else self.group_size
        self.n_groups = -(-self.cols // self.g)
        self.codes = np.zeros((self.rows, self.cols), dtype=np.int64)
        self.pre = np.zeros((self.rows, self.cols))           # w/scale + zero
        self.scales = np.zeros((self.n_groups, self.rows))
        self.zeros = np.zeros((self.n_groups, self.rows), dtype=np.int64)
        self.zero_pre = np.zeros((self.n_groups, self.rows))
        self.code_div = []     # (row, col, |v - midpoint|, |code_a - code_b|)
        self.zero_div = []     # (group, row, |v - midpoint|, |zero_a - zero_b|)
        self._scale = self._zero = None

    @staticmethod
    def _midpoint_gap(v, a, b):
        return np.abs(v - 0.5 * (a + b)), np.abs(a - b)

    def __call__(self, q: int, Wp: np.ndarray) -> np.ndarray:
        if q % self.g == 0:
            gi = q // self.g
            scale, zero, zval = fit_minmax(Wp[:, q:q + self.g], self.maxq)
            if self.forced_zeros is not None:
                fz = self.forced_zeros[gi].astype(np.float64)
                bad = np.nonzero(fz != zero)[0]
                gap, dist = self._midpoint_gap(zval[bad], zero[bad], fz[bad])
                self.zero_div += [(gi, int(r), float(g_), float(d_)) for r, g_, d_ in zip(bad, gap, dist)]
                zero = fz
            self._scale, self._zero = scale, zero
            self.scales[gi], self.zeros[gi], self.zero_pre[gi] = scale, zero, zval
        v = Wp[:, q] / self._scale + self._zero
        code = np.clip(np.rint(v), 0, self.maxq)
        if self.forced_codes is not None:
            fc = self.forced_codes[:, q].astype(np.float64)
            bad = np.nonzero(fc != code)[0]
            gap, dist = self._midpoint_gap(v[bad], code[bad], fc[bad])
            self.code_div += [(int(r), q, float(g_), float(d_)) for r, g_, d_ in zip(bad, gap, dist)]
            code = fc
        self.pre[:, q] = v
        self.codes[:, q] = code
        return self._scale * (code - self._zero)


def ref_quantize_layer(W: np.ndarray, dtype: str, prep: dict, bits: int = 4,
                       group_size: int = 128, block_size: int = 128,
                       forced_codes: np.ndarray | None = None,
                       forced_zeros: np.ndarray | None = None):
    """GPTQ of one layer given the output of :func:`ref_prepare_hinv`.

    W [d_out, d_in] (stored dtype) -> codes [d_out, d_in] in ORIGINAL column order,
    scales / zeros [n_groups, d_out] (groups formed in processing order), g_idx
    [d_in] (group of each original column, [ARCH] "Groups, act-order and other
    knobs"), perm, and the dequantized What in original order.
    ``forced_codes`` (original order) / ``forced_zeros`` switch on the replay.
    """
    U, perm, dead = prep["U"], prep["perm"], prep["dead"]
    Wf = widen(W, dtype)
    rows, cols = Wf.shape
    Wf[:, dead] = 0.0
    Wp = Wf[:, perm].copy()
    fc = None if forced_codes is None else np.asarray(forced_codes)[:, perm]
    grid = MinMaxGrid(rows, cols, bits, group_size, fc, forced_zeros)
    What_p = gptq_sweep(Wp, U, block_size, grid)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(cols)
    codes = grid.codes[:, inv].astype(np.uint8)
    g_idx = (inv // grid.g).astype(np.int32)
    return dict(codes=codes, scales=grid.scales, zeros=grid.zeros.astype(np.uint8),
                g_idx=g_idx, perm=perm, What=What_p[:, inv], grid=grid)


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


# ------------------------------------------------------------------- whole layer

def ref_gptq_layer(W: np.ndarray, X_chunks, dtype: str, bits: int = 4, group_size: int = 128,
                   block_size: int = 128, damp: float = 0.01, act_order: bool = False,
                   timings: dict | None = None):
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
    res = ref_quantize_layer(W, dtype, prep, bits, group_size, block_size)
    t3 = time.perf_counter()
    if timings is not None:
        timings.update(hessian=t1 - t0, prepare=t2 - t1, quantize=t3 - t2)
    res.update(H=H, n_seen=n, prep=prep)
    return res
