"""The page's 4x4 worked example as a pin of the oracle's sweep, loss and rounding.

Fixture: tests/golden/worked_example_4x4.json ("Same Ruler, Smarter Placement:
GPTQ", sections 1.11 and 2).  The page's grid is symmetric per input column with
scale max|column| / 7; it is used here as a test-only grid through the oracle's
generic sweep (the page's scale max|w| / 7 with codes in [-8, 7]).  The page compensates with unconditioned rows of its inverse, which
coincides with GPTQ for the first column only, so the checks are: the column-0 step,
the codes of columns 0-2 (which the conditional procedure reproduces), the RTN and
naive per-tensor losses, and the true output y.
"""
import json
import os

import numpy as np
import pytest

from oracle import gptq_ref as R

FIX = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example_4x4.json")))
W = np.array(FIX["W"])
SX = np.array(FIX["s_X"])
H = np.array(FIX["H"])


def sym_column_grid(codes_out):
    def quant(q, Wp):
        delta = np.max(np.abs(Wp[:, q])) / 7.0
        c = np.clip(np.rint(Wp[:, q] / delta), -8, 7)
        codes_out[q] = c.astype(int).tolist()
        return c * delta
    return quant


def test_true_output():
    np.testing.assert_allclose(W @ SX, FIX["y"], atol=5e-4)


def test_printed_inverse_is_the_inverse_hessian():
    np.testing.assert_allclose(np.linalg.inv(H), FIX["Hinv_2dp"], atol=0.005)


def test_column_zero_step_and_first_codes():
    U = R.ref_prepare_hinv(H, damp=0.0)["U"]
    codes = {}
    Wp = W.copy()
    quant = sym_column_grid(codes)
    # the first column through the oracle's sweep (a one-column problem)
    R.obs_sweep(Wp[:, :1].copy(), U[:1, :1], quant)   # fills codes[0]
    Wstep = W.copy()
    Wq0 = np.array(codes[0]) * np.max(np.abs(W[:, 0])) / 7.0
    err = (W[:, 0] - Wq0) / U[0, 0]
    Wstep[:, 1:] -= np.outer(err, U[0, 1:])
    Wstep[:, 0] = Wq0
    np.testing.assert_allclose(Wstep, FIX["W_after_col0"], atol=2e-4)
    # full conditional sweep: the first three columns keep the page's codes
    codes = {}
    R.obs_sweep(W.copy(), U, sym_column_grid(codes))
    assert [codes[0], codes[1], codes[2]] == FIX["codes_cols_0_1_2"]


def test_rtn_and_naive_losses():
    Hx = 2.0 * np.outer(SX, SX)                        # one calibration token x = s_X
    d = np.max(np.abs(W), axis=0) / 7.0
    rtn = np.clip(np.rint(W / d), -8, 7) * d
    assert R.ref_layer_loss(W.astype(np.float32), "f32", rtn, Hx) == pytest.approx(FIX["loss_rtn_per_column"], abs=6e-4)
    dt = np.max(np.abs(W)) / 7.0
    naive = np.clip(np.rint(W / dt), -8, 7) * dt
    assert R.ref_layer_loss(W.astype(np.float32), "f32", naive, Hx) == pytest.approx(FIX["loss_naive_per_tensor"], abs=6e-4)
