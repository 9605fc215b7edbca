"""Pins of the oracle's column sweep, grid and loss (CPU only).

The oracle (unblocked sweep on the rows of U) is checked against formulations it shares
no code with: explicit-inverse OBS downdates, the lazy-batch sweep of "Same Ruler,
Smarter Placement: GPTQ" 1.8 at several block sizes, Babai's nearest plane on the
Hessian lattice ("04 — GPTQ: ...", section 4), and round-to-nearest when H is
diagonal.  Exact rounding ties pin the order of rounding and zero point ("GPTQ
Architecture, in depth", "The algorithm in code": the quotient is rounded, then the
zero point is added).  H -> cH invariance follows from the relative damping of 1.6.
"""
import numpy as np
import pytest

from oracle import gptq_ref as R
from tests import xcheck


def problem(seed, d_out, d_in, n, dead=()):
    rng = np.random.default_rng(seed)
    X = (rng.standard_normal((n, d_in)) * np.exp(rng.standard_normal(d_in))).astype(np.float32)
    X[:, list(dead)] = 0.0
    W = (0.02 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    H, _ = R.ref_accumulate_hessian(X, "f32")
    return W, X, H


def processing_weights(W, prep):
    Wp = W.astype(np.float64)
    Wp[:, prep["dead"]] = 0.0
    return Wp[:, prep["perm"]]


CASES = [
    # seed, d_out, d_in, n, bits, group, act_order, dead, sym
    (0, 8, 16, 64, 4, -1, False, (), False),
    (1, 12, 32, 80, 3, 16, True, (), False),
    (2, 6, 48, 40, 4, 16, True, (3, 17), False),
    (3, 16, 64, 200, 4, 32, False, (), False),
    (4, 9, 24, 30, 3, -1, True, (0,), False),
    (5, 20, 96, 300, 4, 32, True, (), False),
    (6, 4, 8, 6, 4, -1, False, (), False),
    (7, 10, 40, 120, 3, 8, True, (39,), False),
    (8, 10, 32, 90, 4, 16, True, (), True),
    (9, 7, 24, 60, 3, -1, False, (5,), True),
    (10, 12, 48, 100, 2, 8, True, (), True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
def test_matches_explicit_inverse_obs_downdates(case):
    seed, d_out, d_in, n, bits, group, act, dead, sym = case
    W, X, H = problem(seed, d_out, d_in, n, dead)
    prep = R.ref_prepare_hinv(H, 0.01, act)
    res = R.ref_quantize_layer(W, "f32", prep, bits, group, sym=sym)
    ref = xcheck.obs_downdate(processing_weights(W, prep), prep["Hp"], bits, group, sym)
    got = res["codes"][:, prep["perm"]]
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("seed,group,sym", [(70, 16, False), (71, 8, True), (72, 32, False), (73, 16, True)])
def test_static_groups_match_explicit_inverse_obs_downdates(seed, group, sym):
    # groups of consecutive ORIGINAL columns, fitted before the sweep, used in permuted order
    W, X, H = problem(seed, 9, 64, 150, dead=(7,))
    prep = R.ref_prepare_hinv(H, 0.01, act_order=True)
    res = R.ref_quantize_layer(W, "f32", prep, 4, group, sym=sym, static_groups=True)
    Wz = W.astype(np.float64)
    Wz[:, prep["dead"]] = 0.0
    fixed = xcheck.static_grids(Wz, prep["perm"], 4, group, sym)
    ref = xcheck.obs_downdate(processing_weights(W, prep), prep["Hp"], 4, group, sym, fixed=fixed)
    assert np.array_equal(res["codes"][:, prep["perm"]], ref)
    # contiguous groups: g_idx is c // g, and the stored grid of each group is its up-front fit
    assert res["g_idx"].tolist() == [c // group for c in range(64)]
    for gi in range(64 // group):
        for r in range(9):
            s, z = xcheck.segment_grid(Wz[r, gi * group:(gi + 1) * group], 4, sym)
            assert res["scales"][gi, r] == pytest.approx(s, rel=1e-15) and res["zeros"][gi, r] == z


@pytest.mark.parametrize("block", [1, 4, 16, 32, 64])
@pytest.mark.parametrize("group,sym", [(16, False), (-1, False), (8, True)])
def test_lazy_batches_give_the_unblocked_result(block, group, sym):
    # "Same Ruler, Smarter Placement: GPTQ" 1.8: batching changes when updates land, not which
    W, X, H = problem(30, 14, 64, 150)
    prep = R.ref_prepare_hinv(H, 0.01, True)
    res = R.ref_quantize_layer(W, "f32", prep, 4, group, sym=sym)
    ref = xcheck.lazy_blocked(processing_weights(W, prep), prep["U"], 4, group, block, sym)
    assert np.array_equal(res["codes"][:, prep["perm"]], ref)


@pytest.mark.parametrize("seed,act", [(10, False), (11, True), (12, True), (13, False)])
def test_matches_babai_nearest_plane_per_row_grid(seed, act):
    d_out, d_in, n, bits = 10, 24, 50, 4 if seed % 2 else 3
    W, X, H = problem(seed, d_out, d_in, n)
    prep = R.ref_prepare_hinv(H, 0.01, act)
    res = R.ref_quantize_layer(W, "f32", prep, bits, -1)
    perm = prep["perm"]
    M = np.vstack([np.sqrt(2.0) * X.astype(np.float64)[:, perm], np.sqrt(prep["lam"]) * np.eye(d_in)])
    ref = xcheck.babai(W.astype(np.float64)[:, perm], M, bits)
    assert np.array_equal(res["codes"][:, perm], ref)


@pytest.mark.parametrize("group,sym", [(-1, False), (8, False), (16, False), (-1, True), (8, True)])
def test_diagonal_hessian_reduces_to_round_to_nearest(group, sym):
    rng = np.random.default_rng(20)
    W = (0.05 * rng.standard_normal((7, 32))).astype(np.float32)
    H = np.diag(np.exp(rng.standard_normal(32)))
    prep = R.ref_prepare_hinv(H, 0.01, act_order=True)
    res = R.ref_quantize_layer(W, "f32", prep, 4, group, sym=sym)
    Wp = W.astype(np.float64)[:, prep["perm"]]
    assert np.array_equal(res["codes"][:, prep["perm"]], xcheck.rtn(Wp, 4, group, sym))


def test_diagonal_hessian_static_groups_is_round_to_nearest_on_original_groups():
    rng = np.random.default_rng(21)
    W = (0.05 * rng.standard_normal((6, 32))).astype(np.float32)
    H = np.diag(np.exp(rng.standard_normal(32)))
    prep = R.ref_prepare_hinv(H, 0.01, act_order=True)
    res = R.ref_quantize_layer(W, "f32", prep, 3, 8, static_groups=True)
    # no compensation: the original-order round-to-nearest codes, whatever the order
    assert np.array_equal(res["codes"], xcheck.rtn(W.astype(np.float64), 3, 8))


def test_exact_rounding_ties_round_the_quotient_before_adding_the_zero():
    # diagonal H: nothing is propagated, so the codes are the grid's own decisions.
    # Row [-1, 14, 2.5, 0]: lo = -1, hi = 14, scale = 15 / 15 = 1, zero = 1.  Column 2 is
    # 2.5 / 1 = 2.5 exactly: round half to even gives 2, plus the zero 1 -> code 3 (rounding
    # 2.5 + 1 = 3.5 instead would give 4).
    W = np.array([[-1.0, 14.0, 2.5, 0.0]], dtype=np.float32)
    prep = R.ref_prepare_hinv(np.diag([1.0, 2.0, 3.0, 4.0]), 0.01, act_order=False)
    res = R.ref_quantize_layer(W, "f32", prep, 4, -1)
    assert res["zeros"][0, 0] == 1 and res["scales"][0, 0] == 1.0
    assert res["codes"][0].tolist() == [0, 15, 3, 1]
    # groups of 4 with an odd zero (3): 0.5 -> 0 + 3 = 3 and 1.5 -> 2 + 3 = 5
    W2 = np.array([[-3.0, 12.0, 0.5, 1.5, 2.0, -1.0, 0.0, 13.0]], dtype=np.float32)
    prep2 = R.ref_prepare_hinv(np.diag(np.arange(1.0, 9.0)), 0.01, act_order=False)
    res2 = R.ref_quantize_layer(W2, "f32", prep2, 4, 4)
    assert res2["zeros"][:, 0].tolist() == [3, 1]
    assert res2["codes"][0, :4].tolist() == [0, 15, 3, 5]
    # second group: lo = -1, hi = 13, scale 14/15 (not exact), zero = round(15/14) = 1
    assert res2["codes"][0, 4:].tolist() == [3, 0, 1, 15]
    # symmetric 4-bit: zero 8, scale = 14 / 7 = 2; 5.0 / 2 = 2.5 -> 2 + 8 = 10, -3 / 2 = -1.5 -> -2 + 8 = 6
    W3 = np.array([[14.0, 5.0, -3.0, -14.0]], dtype=np.float32)
    res3 = R.ref_quantize_layer(W3, "f32", prep, 4, -1, sym=True)
    assert res3["zeros"][0, 0] == 8 and res3["scales"][0, 0] == 2.0
    assert res3["codes"][0].tolist() == [15, 10, 6, 1]


def test_hessian_scale_invariance():
    W, X, H = problem(31, 12, 48, 100)
    a = R.ref_quantize_layer(W, "f32", R.ref_prepare_hinv(H, 0.01, True), 4, 16)
    b = R.ref_quantize_layer(W, "f32", R.ref_prepare_hinv(H * 1e-3, 0.01, True), 4, 16)
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["zeros"], b["zeros"])


def test_loss_is_the_output_error_on_the_calibration_set():
    W, X, H = problem(32, 9, 32, 70, dead=(5,))
    res = R.ref_quantize_layer(W, "f32", R.ref_prepare_hinv(H, 0.01, True), 3, 16)
    direct = np.sum(((W.astype(np.float64) - res["What"]) @ X.astype(np.float64).T) ** 2)
    assert R.ref_layer_loss(W, "f32", res["What"], H) == pytest.approx(direct, rel=1e-10)
    # dequantisation from codes / scales / zeros / g_idx reproduces What
    np.testing.assert_allclose(R.ref_dequantize(res["codes"], res["scales"], res["zeros"], res["g_idx"]),
                               res["What"], rtol=1e-13, atol=1e-15)
    st = R.ref_quantize_layer(W, "f32", R.ref_prepare_hinv(H, 0.01, True), 3, 16, sym=True, static_groups=True)
    np.testing.assert_allclose(R.ref_dequantize(st["codes"], st["scales"], st["zeros"], st["g_idx"]),
                               st["What"], rtol=1e-13, atol=1e-15)


def test_gptq_beats_rtn_on_average():
    wins = []
    for seed in range(8):
        W, X, H = problem(40 + seed, 16, 64, 256)
        prep = R.ref_prepare_hinv(H, 0.01, True)
        g = R.ref_quantize_layer(W, "f32", prep, 4, 32)
        diagH = np.diag(np.diag(H))
        r = R.ref_quantize_layer(W, "f32", R.ref_prepare_hinv(diagH, 0.01, True), 4, 32)
        wins.append(R.ref_layer_loss(W, "f32", g["What"], H) < R.ref_layer_loss(W, "f32", r["What"], H))
    assert sum(wins) >= 7


def test_grid_edge_cases():
    seg = np.array([[0.3, 0.1, 0.2], [0.0, 0.0, 0.0], [-0.2, -0.4, -0.1], [-1.0, 0.5, 2.0]])
    s, z, zv = R.UniformGrid(4).fit(seg)
    np.testing.assert_allclose(s, [0.3 / 15, 1e-8, 0.4 / 15, 3.0 / 15])
    assert z.tolist() == [0.0, 0.0, 15.0, 5.0]
    np.testing.assert_allclose(zv, [0.0, 0.0, 15.0, 5.0])
    s2, z2, _ = R.UniformGrid(3, sym=True).fit(seg)
    np.testing.assert_allclose(s2, [0.3 / 3, 1e-8, 0.4 / 3, 2.0 / 3])
    assert z2.tolist() == [4.0] * 4
    # clamping at both ends
    c, _ = R.UniformGrid(4).code(np.array([-5.0, 0.0, 5.0]), np.ones(3), np.full(3, 2.0))
    assert c.tolist() == [0.0, 2.0, 7.0]


def test_group_index_and_processing_order():
    W, X, H = problem(50, 5, 32, 64)
    prep = R.ref_prepare_hinv(H, 0.01, True)
    res = R.ref_quantize_layer(W, "f32", prep, 4, 8)
    perm = prep["perm"]
    for pos, c in enumerate(perm):
        assert res["g_idx"][c] == pos // 8
    assert res["scales"].shape == (4, 5) and res["zeros"].shape == (4, 5)


def test_replay_with_own_decisions_has_no_divergence_and_flags_planted_flip():
    W, X, H = problem(60, 8, 32, 64)
    prep = R.ref_prepare_hinv(H, 0.01, True)
    a = R.ref_quantize_layer(W, "f32", prep, 4, 16)
    b = R.ref_quantize_layer(W, "f32", prep, 4, 16, forced_codes=a["codes"], forced_zeros=a["zeros"])
    assert b["grid"].code_div == [] and b["grid"].zero_div == []
    np.testing.assert_array_equal(a["codes"], b["codes"])
    bad = a["codes"].copy()
    c = int(prep["perm"][3])
    bad[2, c] = bad[2, c] + 1 if bad[2, c] < 15 else bad[2, c] - 1
    r = R.ref_quantize_layer(W, "f32", prep, 4, 16, forced_codes=bad, forced_zeros=a["zeros"])
    divs = r["grid"].code_div
    # the planted flip is the first divergence, far from a midpoint; its error then
    # re-routes the rest of that row only (rows are independent given U)
    assert divs[0][:2] == (2, 3) and divs[0][2] > 1e-5
    assert all(dv[0] == 2 for dv in divs)


def test_fp16_widening_is_exact():
    bits = np.array([[0x3C00, 0xC000, 0x3C01, 0x0001, 0x7BFF, 0x8400]], dtype=np.uint16)
    got = R.widen(bits, "f16")
    assert got.tolist() == [[1.0, -2.0, 1.0 + 2 ** -10, 2.0 ** -24, 65504.0, -(2.0 ** -14)]]
