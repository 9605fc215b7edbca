"""Pins of the oracle's dead-input fix, ActOrder, damping and U (CPU only).

Pages: "Same Ruler, Smarter Placement: GPTQ" 1.6 (damping: eigenvalues shift by
lambda, [H_damp^-1]_qq <= 1/lambda), 1.7 (2x2 closed form; u_qq^2 is the conditional
inverse-Hessian diagonal after earlier columns are eliminated), 1.9 (ActOrder);
"GPTQ Architecture, in depth", "The algorithm in code" (dead inputs, damping mean).
"""
import numpy as np
import pytest

from oracle import gptq_ref as R


def spd(d, seed, n=None):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n or 3 * d, d)) * np.exp(rng.standard_normal(d))
    return 2.0 * X.T @ X


def test_two_by_two_closed_form():
    H = np.array([[3.0, 1.2], [1.2, 2.0]])
    damp = 0.05
    lam = damp * (3.0 + 2.0) / 2
    Hd = H + lam * np.eye(2)
    det = Hd[0, 0] * Hd[1, 1] - Hd[0, 1] ** 2
    a, b, c = Hd[1, 1] / det, -Hd[0, 1] / det, Hd[0, 0] / det   # H_damp^-1 = [[a, b], [b, c]]
    U = R.ref_prepare_hinv(H, damp)["U"]
    assert U[1, 0] == 0.0
    np.testing.assert_allclose(U[0, 0], np.sqrt(a), rtol=1e-14)
    np.testing.assert_allclose(U[0, 1], b / np.sqrt(a), rtol=1e-13)
    np.testing.assert_allclose(U[1, 1], np.sqrt(c - b * b / a), rtol=1e-13)
    np.testing.assert_allclose(U[0, 1] / U[0, 0], b / a, rtol=1e-13)


def test_rows_of_U_are_the_conditional_inverse_after_downdates():
    H = spd(12, 1)
    p = R.ref_prepare_hinv(H, 0.01)
    U = p["U"]
    Hinv = np.linalg.inv(p["Hp"])
    for q in range(12):
        # conditional inverse of the remaining problem: Schur complement downdates
        np.testing.assert_allclose(U[q, q] ** 2, Hinv[q, q], rtol=1e-10)
        np.testing.assert_allclose(U[q, q + 1:] / U[q, q], Hinv[q, q + 1:] / Hinv[q, q], rtol=1e-8, atol=1e-12)
        Hinv = Hinv - np.outer(Hinv[:, q], Hinv[q, :]) / Hinv[q, q]


def test_U_is_an_upper_factor_of_the_damped_inverse():
    H = spd(40, 2)
    p = R.ref_prepare_hinv(H, 0.01, act_order=True)
    U = p["U"]
    assert np.all(np.tril(U, -1) == 0) and np.all(np.diag(U) > 0)
    np.testing.assert_allclose(U.T @ U @ p["Hp"], np.eye(40), atol=1e-9)


def test_damping_shifts_eigenvalues_and_bounds_the_inverse_diagonal():
    H = spd(16, 3, n=8)                 # rank-deficient: n < d
    p = R.ref_prepare_hinv(H, 0.01)
    lam = p["lam"]
    assert lam == pytest.approx(0.01 * np.mean(np.diag(H)), rel=1e-15)
    ev0 = np.linalg.eigvalsh(H)
    ev1 = np.linalg.eigvalsh(p["Hp"])
    np.testing.assert_allclose(ev1, ev0 + lam, atol=1e-9 * ev0.max())
    U = p["U"]
    inv_diag = np.sum(U * U, axis=0)    # [U^T U]_qq
    assert np.all(inv_diag <= 1.0 / lam * (1 + 1e-12))


def test_actorder_is_descending_with_ties_in_index_order_and_dead_inputs():
    rng = np.random.default_rng(4)
    X = rng.integers(-9, 10, size=(40, 7)).astype(np.float64)
    X[:, [2, 5]] = 0.0                  # two inputs never active
    X[:, 6] = -X[::-1, 3]               # same energy as input 3: an exact tie
    H = 2.0 * X.T @ X
    assert H[3, 3] == H[6, 6]
    p = R.ref_prepare_hinv(H, 0.01, act_order=True)
    assert p["dead"].tolist() == [False, False, True, False, False, True, False]
    key = np.diag(H).copy()
    key[[2, 5]] = 1.0
    perm = p["perm"].tolist()
    # brute-force: a column precedes another iff its key is larger, or equal with a lower index
    for a in range(7):
        for b in range(a + 1, 7):
            i, j = perm[a], perm[b]
            assert key[i] > key[j] or (key[i] == key[j] and i < j)
    assert perm.index(3) < perm.index(6) and perm.index(2) < perm.index(5)
    # the fixed diagonal enters the damping mean
    assert p["lam"] == pytest.approx(0.01 * key.mean(), rel=1e-15)


def test_not_spd_is_reported():
    H = spd(10, 5, n=4)
    with pytest.raises(R.NotSPD):
        R.ref_prepare_hinv(H, 0.0)
    H2 = spd(6, 6)
    H2[1, 1] = -abs(H2[1, 1])
    with pytest.raises(R.NotSPD):
        R.ref_prepare_hinv(H2, 0.01)


def test_reversed_factorisation_gives_the_same_U():
    # H_p = Ut Ut^T with Ut upper (Cholesky of the index-reversed matrix), U = Ut^-1.
    H = spd(30, 7)
    p = R.ref_prepare_hinv(H, 0.01)
    J = np.arange(30)[::-1]
    L = np.linalg.cholesky(p["Hp"][np.ix_(J, J)])
    U2 = np.linalg.inv(L)[np.ix_(J, J)]
    np.testing.assert_allclose(U2, p["U"], rtol=1e-9, atol=1e-12)


def test_column_order_from_the_diagonal_alone():
    # dead inputs (zero diagonal) count as 1; descending; ties keep the original order
    diag = np.array([2.0, 0.0, 5.0, 1.0, 2.0, 0.0, 7.0])
    perm, dead, fixed = R.ref_column_order(diag, act_order=True)
    assert perm.tolist() == [6, 2, 0, 4, 1, 3, 5]
    assert dead.tolist() == [False, True, False, False, False, True, False]
    assert fixed.tolist() == [2.0, 1.0, 5.0, 1.0, 2.0, 1.0, 7.0]
    perm0, _, _ = R.ref_column_order(diag, act_order=False)
    assert perm0.tolist() == list(range(7))
