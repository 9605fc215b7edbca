"""Pins of the oracle's Hessian accumulation (CPU only).

H = 2 X X^T ("Same Ruler, Smarter Placement: GPTQ", 1.4), accumulated over
calibration batches ("GPTQ Architecture, in depth", "The algorithm in code").
"""
import numpy as np

from oracle import gptq_ref as R
from post_weight_quantization_03_amd import synth


def brute_hessian(X):
    n, d = len(X), len(X[0])
    H = [[0 for _ in range(d)] for _ in range(d)]
    for t in range(n):
        for i in range(d):
            for j in range(d):
                H[i][j] += 2 * X[t][i] * X[t][j]
    return np.array(H, dtype=np.float64)


def test_integer_inputs_match_brute_force_exactly():
    rng = np.random.default_rng(5)
    X = rng.integers(-7, 8, size=(13, 6)).astype(np.float32)
    H, n = R.ref_accumulate_hessian(X, "f32")
    assert n == 13
    assert np.array_equal(H, brute_hessian(X.astype(int).tolist()))


def test_chunked_accumulation_equals_one_shot():
    rng = np.random.default_rng(6)
    X = rng.integers(-5, 6, size=(37, 8)).astype(np.float32)
    H1, n1 = R.ref_accumulate_hessian(X, "f32")
    H2, n2 = None, 0
    for a, b in [(0, 5), (5, 6), (6, 30), (30, 37)]:
        H2, n2 = R.ref_accumulate_hessian(X[a:b], "f32", H2, n2, rows_per_step=3)
    assert n1 == n2 == 37
    assert np.array_equal(H1, H2)


def test_diagonal_is_twice_the_channel_energy_and_one_hot_closed_form():
    # one-hot tokens: channel c fires k_c times with value v_c -> H = diag(2 k_c v_c^2)
    counts = [3, 0, 1, 5]
    vals = [0.5, 0.0, -2.0, 1.25]
    rows = []
    for c, (k, v) in enumerate(zip(counts, vals)):
        for _ in range(k):
            r = [0.0] * 4
            r[c] = v
            rows.append(r)
    X = np.array(rows, dtype=np.float32)
    H, _ = R.ref_accumulate_hessian(X, "f32")
    assert np.array_equal(H, np.diag([2 * k * v * v for k, v in zip(counts, vals)]))


def test_bf16_widening_is_exact():
    bits = np.array([[0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x4049]], dtype=np.uint16)
    got = R.widen(bits, "bf16")
    assert got.tolist() == [[1.0, -2.0, 1.0078125, 0.0, -0.0, 3.140625]]


def test_bf16_rounding_of_generator_is_nearest_even():
    a = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -3.0], dtype=np.float32)
    # ties go to even mantissa: 1+2^-8 -> 1.0 ; 1+3*2^-8 -> 1+2^-6 ; below half -> 1.0
    back = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a))
    assert back.tolist() == [1.0, 1.0 + 2 ** -6, 1.0, -3.0]


def test_generator_is_deterministic_and_chunkable():
    spec = synth.scaled("attn_proj", d_out=16, d_in=128, n_tokens=300, seq_len=128)
    X1 = synth.make_activations(spec, threads=1)
    X2 = synth.make_activations(spec, threads=4)
    assert np.array_equal(X1, X2)
    assert X1.shape == (300, 128) and X1.dtype == np.uint16
    s = synth.make_channel_scales(spec)
    assert np.array_equal(X1[128:256], synth.make_sequence(spec, 1, 128, s))


def test_channel_energy_and_entry_blocks_match_brute_force_exactly():
    # integer inputs: every product and sum is exact in fp64, so equality is exact
    rng = np.random.default_rng(7)
    X = rng.integers(-9, 10, size=(29, 7)).astype(np.float32)
    Hb = brute_hessian(X.astype(int).tolist())
    assert np.array_equal(R.ref_channel_energy(X, "f32", rows_per_step=4), np.diag(Hb))
    rows, cols = np.array([6, 0, 3]), np.array([1, 1, 5, 2])
    assert np.array_equal(R.ref_hessian_entries(X, "f32", rows, cols, rows_per_step=5), Hb[np.ix_(rows, cols)])


def test_channel_energy_of_bf16_inputs_equals_the_hessian_diagonal():
    spec = synth.scaled("attn_proj", d_out=8, d_in=64, n_tokens=3000, seq_len=1000)
    X = synth.make_activations(spec, 0)
    H, _ = R.ref_accumulate_hessian(X, "bf16", rows_per_step=700)
    np.testing.assert_allclose(R.ref_channel_energy(X, "bf16", rows_per_step=500), np.diag(H), rtol=1e-14)
