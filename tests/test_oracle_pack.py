"""Pins of the oracle's checkpoint packing ("04 — GPTQ: ...", section 8;
"GPTQ Architecture, in depth", "Packing, tooling and serving")."""
import numpy as np
import pytest

from oracle import gptq_ref as R


def test_nibble_order_low_first():
    codes = np.arange(16, dtype=np.uint8).reshape(1, 16).repeat(8, axis=0)   # d_out=8, d_in=16
    zeros = np.array([[1, 2, 3, 4, 5, 6, 7, 8]], dtype=np.uint8)
    qw, qz, sc = R.ref_pack_int4(codes, np.ones((1, 8)), zeros)
    assert qw.shape == (2, 8) and qz.shape == (1, 1)
    assert qw.view(np.uint32)[0, 0] == 0x76543210 and qw.view(np.uint32)[1, 3] == 0xFEDCBA98
    assert qz.view(np.uint32)[0, 0] == 0x87654321


def test_round_trip_and_fp16_scales():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 16, size=(24, 64)).astype(np.uint8)
    zeros = rng.integers(0, 16, size=(4, 24)).astype(np.uint8)
    scales = rng.random((4, 24)) * 1e-2
    qw, qz, sc = R.ref_pack_int4(codes, scales, zeros)
    c2, z2 = R.ref_unpack_int4(qw, qz)
    assert np.array_equal(c2, codes) and np.array_equal(z2, zeros)
    assert sc.dtype == np.float16
    np.testing.assert_array_equal(sc, scales.astype(np.float32).astype(np.float16))


def test_checkpoint_bytes_of_a_4096_square_layer_g128():
    d_out = d_in = 4096
    g = 128
    qweight = (d_in // 8) * d_out * 4
    qzeros = (d_in // g) * (d_out // 8) * 4
    scales = (d_in // g) * d_out * 2
    g_idx = d_in * 4
    total = qweight + qzeros + scales + g_idx
    # the page's own formula: out*in/2 + out*in/g*2 + out*in/(g*2) + in*4
    assert total == d_out * d_in // 2 + d_out * d_in // g * 2 + d_out * d_in // (g * 2) + d_in * 4 == 8732672
    assert round(8 * total / (d_out * d_in), 3) == 4.164


def test_w4a16_product_by_brute_force():
    # Y[m, o] = sum_c x[m, c] * s[g(c), o] * (q[o, c] - z[g(c), o]), written out element by
    # element from the bit layout (nibble k of word i is input 8 i + k of output o)
    rng = np.random.default_rng(3)
    d_out, d_in, g, m = 16, 32, 8, 3
    qweight = rng.integers(0, 2 ** 31, size=(d_in // 8, d_out), dtype=np.int64).astype(np.int32)
    qzeros = rng.integers(0, 2 ** 31, size=(d_in // g, d_out // 8), dtype=np.int64).astype(np.int32)
    scales = (rng.random((d_in // g, d_out)) * 0.1).astype(np.float16)
    g_idx = rng.permutation(np.arange(d_in) // g).astype(np.int32)      # scattered groups (act-order)
    X = rng.standard_normal((m, d_in)).astype(np.float32)
    got = R.ref_w4a16_matmul(X, "f32", qweight, qzeros, scales, g_idx)
    qw, qz = qweight.view(np.uint32), qzeros.view(np.uint32)
    for mi in range(m):
        for o in range(d_out):
            acc = 0.0
            for c in range(d_in):
                q = (int(qw[c // 8, o]) >> (4 * (c % 8))) & 15
                gi = int(g_idx[c])
                z = (int(qz[gi, o // 8]) >> (4 * (o % 8))) & 15
                acc += float(X[mi, c]) * float(scales[gi, o]) * (q - z)
            assert got[mi, o] == pytest.approx(acc, rel=1e-12, abs=1e-12)


def test_w4a16_product_of_a_packed_layer_equals_the_dequantized_weights():
    # pack -> serve round trip: the product from the checkpoint equals X What^T with the
    # scales rounded to fp16 as the checkpoint stores them
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 16, size=(24, 64)).astype(np.uint8)
    zeros = rng.integers(0, 16, size=(4, 24)).astype(np.uint8)
    scales = rng.random((4, 24)) * 1e-2
    g_idx = (np.arange(64) // 16).astype(np.int32)
    qw, qz, sf = R.ref_pack_int4(codes, scales, zeros)
    X = rng.standard_normal((5, 64)).astype(np.float32)
    What = R.ref_dequantize(codes, sf.astype(np.float64), zeros, g_idx)
    np.testing.assert_allclose(R.ref_w4a16_matmul(X, "f32", qw, qz, sf, g_idx), X.astype(np.float64) @ What.T,
                               rtol=1e-13, atol=1e-15)
