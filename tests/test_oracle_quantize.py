"""Pins of the oracle's column sweep, grid and loss (CPU only).

The oracle (Cholesky rows + lazy blocks) is checked against formulations it shares
no code with: explicit-inverse OBS downdates, Babai's nearest plane on the Hessian
lattice ("04 — GPTQ: ...", section 4), and round-to-nearest when H is diagonal.
Block-size invariance restates "Same Ruler, Smarter Placement: GPTQ" 1.8 (lazy
batching changes when updates land, not which); H -> cH invariance follows from the
relative damping of 1.6.
"""
import itertools

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


CASES = [
    # seed, d_out, d_in, n, bits, group, act_order, dead
    (0, 8, 16, 64, 4, -1, False, ()),
    (1, 12, 32, 80, 3, 16, True, ()),
    (2, 6, 48, 40, 4, 16, True, (3, 17)),
    (3, 16, 64, 200, 4, 32, False, ()),
    (4, 9, 24, 30, 3, -1, True, (0,)),
    (5, 20, 96, 300, 4, 32, True, ()),
    (6, 4, 8, 6, 4, -1, False, ()),
    (7, 10, 40, 120, 3, 8, True, (39,)),
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
def test_matches_explicit_inverse_obs_downdates(case):
    seed, d_out, d_in, n, bits, group, act, dead = case
    W, X, H = problem(seed, d_out, d_in, n, dead)
    prep = R.ref_prepare_hinv(H, 0.01, act)
    res = R.ref_quantize_layer(W, "f32", prep, bits, group, block_size=16)
    Wp = W.astype(np.float64)
    Wp[:, prep["dead"]] = 0.0
    Wp = Wp[:, prep["perm"]]
    ref = xcheck.obs_downdate(Wp, prep["Hp"], bits, group)
    got = res["codes"][:, prep["perm"]]
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("seed,act", [(10, False), (11, True), (12, True), (13, False)])
def test_matches_babai_nearest_plane_per_row_grid(seed, act):
    d_out, d_in, n, bits = 10, 24, 50, 4 if seed % 2 else 3
    W, X, H = problem(seed, d_out, d_in, n)
    prep = R.ref_prepare_hinv(H, 0.01, act)
    res = R.ref_quantize_layer(W, "f32", prep, bits, -1, block_size=8)
    perm = prep["perm"]
    M = np.vstack([np.sqrt(2.0) * X.astype(np.float64)[:, perm], np.sqrt(prep["lam"]) * np.eye(d_in)])
    ref = xcheck.babai(W.astype(np.float64)[:, perm], M, bits)
    assert np.array_equal(res["codes"][:, perm], ref)


@pytest.mark.parametrize("group", [-1, 8, 16])
def test_diagonal_hessian_reduces_to_round_to_nearest(group):
    rng = np.random.default_rng(20)
    W = (0.05 * rng.standard_normal((7, 32))).astype(np.float32)
    H = np.diag(np.exp(rng.standard_normal(32)))
    prep = R.ref_prepare_hinv(H, 0.01, act_order=True)
    res = R.ref_quantize_layer(W, "f32", prep, 4, group, block_size=8)
    Wp = W.astype(np.float64)[:, prep["perm"]]
    assert np.array_equal(res["codes"][:, prep["perm"]], xcheck.rtn(Wp, 4, group))


def test_block_size_does_not_change_the_result():
    W, X, H = problem(30, 14, 64, 150)
    prep = R.ref_prepare_hinv(H, 0.01, True)
    outs = [R.ref_quantize_layer(W, "f32", prep, 4, 16, block_size=b) for b in (1, 16, 32, 64, 128)]
    for o in outs[1:]:
        assert np.array_equal(o["codes"], outs[0]["codes"])
        np.testing.assert_allclose(o["scales"], outs[0]["scales"], rtol=1e-12)


def test_hessian_scale_invariance():
    W, X, H = problem(31, 12, 48, 100)
    a = R.ref_quantize_layer(W, "f32", R.ref_prepare_hinv(H, 0.01, True), 4, 16, 16)
    b = R.ref_quantize_layer(W, "f32", R.ref_prepare_hinv(H * 1e-3, 0.01, True), 4, 16, 16)
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["zeros"], b["zeros"])


def test_loss_is_the_output_error_on_the_calibration_set():
    W, X, H = problem(32, 9, 32, 70, dead=(5,))
    res = R.ref_quantize_layer(W, "f32", R.ref_prepare_hinv(H, 0.01, True), 3, 16, 16)
    direct = np.sum(((W.astype(np.float64) - res["What"]) @ X.astype(np.float64).T) ** 2)
    assert R.ref_layer_loss(W, "f32", res["What"], H) == pytest.approx(direct, rel=1e-10)
    # dequantisation from codes / scales / zeros / g_idx reproduces What
    np.testing.assert_allclose(R.ref_dequantize(res["codes"], res["scales"], res["zeros"], res["g_idx"]),
                               res["What"], rtol=1e-13, atol=1e-15)


def test_gptq_beats_rtn_on_average():
    wins = []
    for seed in range(8):
        W, X, H = problem(40 + seed, 16, 64, 256)
        prep = R.ref_prepare_hinv(H, 0.01, True)
        g = R.ref_quantize_layer(W, "f32", prep, 4, 32, 32)
        Wp = W.astype(np.float64)[:, prep["perm"]]
        diagH = np.diag(np.diag(H))
        r = R.ref_quantize_layer(W, "f32", R.ref_prepare_hinv(diagH, 0.01, True), 4, 32, 32)
        wins.append(R.ref_layer_loss(W, "f32", g["What"], H) < R.ref_layer_loss(W, "f32", r["What"], H))
    assert sum(wins) >= 7


def test_grid_edge_cases():
    Wg = np.array([[0.3, 0.1, 0.2], [0.0, 0.0, 0.0], [-0.2, -0.4, -0.1], [-1.0, 0.5, 2.0]])
    s, z, zv = R.fit_minmax(Wg, 15)
    np.testing.assert_allclose(s, [0.3 / 15, 1e-8, 0.4 / 15, 3.0 / 15])
    assert z.tolist() == [0.0, 0.0, 15.0, 5.0]


def test_group_index_and_processing_order():
    W, X, H = problem(50, 5, 32, 64)
    prep = R.ref_prepare_hinv(H, 0.01, True)
    res = R.ref_quantize_layer(W, "f32", prep, 4, 8, 8)
    perm = prep["perm"]
    for pos, c in enumerate(perm):
        assert res["g_idx"][c] == pos // 8
    assert res["scales"].shape == (4, 5) and res["zeros"].shape == (4, 5)


def test_replay_with_own_decisions_has_no_divergence_and_flags_planted_flip():
    W, X, H = problem(60, 8, 32, 64)
    prep = R.ref_prepare_hinv(H, 0.01, True)
    a = R.ref_quantize_layer(W, "f32", prep, 4, 16, 16)
    b = R.ref_quantize_layer(W, "f32", prep, 4, 16, 16, forced_codes=a["codes"], forced_zeros=a["zeros"])
    assert b["grid"].code_div == [] and b["grid"].zero_div == []
    np.testing.assert_array_equal(a["codes"], b["codes"])
    bad = a["codes"].copy()
    c = int(prep["perm"][3])
    bad[2, c] = bad[2, c] + 1 if bad[2, c] < 15 else bad[2, c] - 1
    r = R.ref_quantize_layer(W, "f32", prep, 4, 16, 16, forced_codes=bad, forced_zeros=a["zeros"])
    divs = r["grid"].code_div
    # the planted flip is the first divergence, far from a midpoint; its error then
    # re-routes the rest of that row only (rows are independent given U)
    assert divs[0][:2] == (2, 3) and divs[0][2] > 1e-5
    assert all(dv[0] == 2 for dv in divs)
