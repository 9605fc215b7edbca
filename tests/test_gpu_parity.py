"""GPU parity: the HIP path through the C ABI against the CPU oracle (MI355X only).

Sizes are chosen so the oracle finishes in seconds while the kernels still see several
tiles and ragged tails (d_out not a multiple of 64, token counts not a multiple of the
32-token stage, d_in not a multiple of the 256-wide Hessian tile).  Acceptance rules are
in tests/parity.py.
"""
import dataclasses
import sys

import numpy as np
import pytest

from oracle import gptq_ref as R
from post_weight_quantization_03_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu


def announce(what):
    print(f"\n[gpu-case] {what}", flush=True)
    sys.stdout.flush()


CASES = {
    # the tiny recipe at its full size: fp32 inputs, one grid per row, natural order
    "tiny_full": synth.config("tiny"),
    "attn_scaled": synth.scaled("attn_proj", d_out=200, d_in=512, n_tokens=5000, seq_len=1024),
    "mlp_up_scaled": synth.scaled("mlp_up", d_out=328, d_in=384, n_tokens=4096, seq_len=1024),
    "mlp_down_scaled": synth.scaled("mlp_down", d_out=128, d_in=640, n_tokens=3000, seq_len=1024),
    "moe_scaled_4bit": synth.scaled("moe", d_out=96, d_in=256, n_tokens=1100, batch=4, seq_len=512),
    "moe_scaled_3bit": synth.scaled("moe", d_out=96, d_in=256, n_tokens=1100, batch=4, seq_len=512, bits=3),
    "group32_bf16": synth.scaled("attn_proj", d_out=72, d_in=256, n_tokens=2000, seq_len=1000, group_size=32),
    "group64_f32": synth.scaled("attn_proj", d_out=40, d_in=384, n_tokens=1500, seq_len=500, group_size=64,
                                dtype="f32"),
    "group16_actorder": synth.scaled("attn_proj", d_out=33, d_in=256, n_tokens=900, seq_len=300, group_size=16),
    "per_row_bf16_actorder": synth.scaled("mlp_up", d_out=64, d_in=256, n_tokens=700, seq_len=700, group_size=-1,
                                          act_order=True),
    "two_bit": synth.scaled("mlp_down", d_out=64, d_in=256, n_tokens=800, seq_len=800, bits=2),
    "eight_bit": synth.scaled("attn_proj", d_out=64, d_in=256, n_tokens=800, seq_len=800, bits=8),
    # rows enough for the other sweep shapes (threads per workgroup, lanes per row):
    # 256 / 4, 512 / 16, 256 / 4 per row, 512 / 4
    "group64_many_rows": synth.scaled("moe", d_out=512, d_in=256, n_tokens=600, batch=32, seq_len=300,
                                      group_size=64),
    "per_row_many_rows": synth.scaled("moe", d_out=520, d_in=256, n_tokens=600, batch=16, seq_len=300,
                                      group_size=-1),
    "per_row_4_lanes": synth.scaled("moe", d_out=520, d_in=256, n_tokens=600, batch=24, seq_len=300,
                                    group_size=-1),
    "group128_4_lanes_512": synth.scaled("moe", d_out=512, d_in=128, n_tokens=400, batch=64, seq_len=200),
    # (the shape per case follows the sweep's cost rule: threads per workgroup, rows per lane)
    # 704 threads at 4 lanes per row, one row per lane (176 rows per workgroup, 8 x 32 = 256
    # workgroups), with groups and with one grid per row
    "group128_4_lanes_704": synth.scaled("moe", d_out=1408, d_in=256, n_tokens=300, batch=32, seq_len=300),
    "per_row_4_lanes_704": synth.scaled("moe", d_out=1408, d_in=256, n_tokens=300, batch=32, seq_len=300,
                                        group_size=-1),
    # 512 threads at 4 lanes per row, two rows per lane (4 x 64 = 256 workgroups of 256 rows)
    "group128_4_lanes_1024": synth.scaled("moe", d_out=1024, d_in=128, n_tokens=300, batch=64, seq_len=300),
    # 704 threads, two rows per lane (352 rows per workgroup, 4 x 64 workgroups), the last
    # workgroup of each expert ragged: its second pass partly past d_out (1300 rows), or its
    # first pass partly and its second wholly (1100 rows, one grid per row)
    "group128_4_lanes_2rows_704": synth.scaled("moe", d_out=1300, d_in=256, n_tokens=300, batch=64, seq_len=300),
    "per_row_4_lanes_2rows_704": synth.scaled("moe", d_out=1100, d_in=256, n_tokens=300, batch=64, seq_len=300,
                                              group_size=-1),
    # fp16 inputs (the f16 matrix-core SYRK, fp16 channel energies and weight permutes)
    "fp16_attn_scaled": synth.scaled("attn_proj", d_out=136, d_in=384, n_tokens=3000, seq_len=1000, dtype="f16"),
    "fp16_moe_scaled": synth.scaled("moe", d_out=64, d_in=256, n_tokens=900, batch=3, seq_len=300, dtype="f16",
                                    bits=3),
    # symmetric grids and static groups ("GPTQ Architecture, in depth", "Groups, act-order and
    # other knobs"), across per-row, every group size and both lane layouts of the sweep
    "sym_g128_actorder": synth.scaled("attn_proj", d_out=200, d_in=512, n_tokens=5000, seq_len=1024, sym=True),
    "sym_per_row_many_rows": synth.scaled("moe", d_out=520, d_in=256, n_tokens=600, batch=16, seq_len=300,
                                          group_size=-1, sym=True),
    "sym_g32_3bit": synth.scaled("mlp_down", d_out=72, d_in=256, n_tokens=1500, seq_len=500, group_size=32, bits=3,
                                 sym=True),
    # the same grids at 4 lanes per row: two rows per lane (1300 rows x 64, ragged last
    # workgroups), and groups of 64 (one row per lane, at most 512 threads)
    "sym_g128_4_lanes_2rows": synth.scaled("moe", d_out=1300, d_in=256, n_tokens=300, batch=64, seq_len=300,
                                           sym=True),
    "group64_4_lanes": synth.scaled("moe", d_out=1000, d_in=256, n_tokens=300, batch=16, seq_len=300,
                                    group_size=64),
    "static_g128_actorder": synth.scaled("attn_proj", d_out=136, d_in=512, n_tokens=4000, seq_len=1000,
                                         static_groups=True),
    "static_g16_sym_f32": synth.scaled("attn_proj", d_out=40, d_in=384, n_tokens=1500, seq_len=500, group_size=16,
                                       dtype="f32", sym=True, static_groups=True),
    "static_g64_moe_many_rows": synth.scaled("moe", d_out=512, d_in=256, n_tokens=600, batch=8, seq_len=300,
                                             group_size=64, static_groups=True),
    "static_no_actorder": synth.scaled("mlp_up", d_out=96, d_in=256, n_tokens=1200, seq_len=600,
                                       static_groups=True),
    # the triangular inverse enqueued beside the factorization (every 8 block columns): 13
    # block columns (ragged doubling groups at two levels), 10 for a batch of two (the blocked
    # Cholesky) and for a batch of four (the left-looking one)
    "inverse_13_blocks": synth.scaled("attn_proj", d_out=64, d_in=1664, n_tokens=4000, seq_len=1000),
    "inverse_10_blocks_batch2": synth.scaled("moe", d_out=64, d_in=1280, n_tokens=3000, batch=2, seq_len=1000),
    "inverse_10_blocks_batch4": synth.scaled("moe", d_out=64, d_in=1280, n_tokens=3000, batch=4, seq_len=1000),
    # 36 block columns: the Cholesky's far updates grouped four panels at a time; lazy updates,
    # trailing updates and the triangular inverse large enough for the split-bf16 products
    # (ragged row tiles: 1944 = 15 x 128 + 24; both B layouts; lower-only output)
    "wide_dense_grouped": synth.scaled("mlp_down", d_out=1944, d_in=4608, n_tokens=6000, seq_len=1000),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layer_parity(name):
    spec = CASES[name]
    announce(f"{name} {spec}")
    Ws, Xs = parity.make_inputs(spec)
    g = parity.run_gpu(spec, Ws, Xs)
    for e in range(spec.batch):
        rep = parity.check_problem(spec, Ws[e], Xs[e], g, e)
        print(name, e, {k: (round(v, 9) if isinstance(v, float) else v) for k, v in rep.items()}, flush=True)


def test_exact_rounding_ties_match_exactly():
    # One-hot calibration tokens give a diagonal H, so nothing is propagated and every code
    # is the grid's own decision on the exact bf16 weight.  The rows are built so that
    # w / scale lands exactly on a half integer with an odd zero point: the quotient is
    # rounded (half to even) before the zero point is added ("GPTQ Architecture, in
    # depth", "The algorithm in code"), which the oracle and the kernel must both do.
    announce("exact rounding ties, diagonal H")
    d_out, d_in = 16, 256
    spec = synth.scaled("attn_proj", d_out=d_out, d_in=d_in, n_tokens=2 * d_in, seq_len=2 * d_in, act_order=False,
                        group_size=-1)
    rng = np.random.default_rng(5)
    X = np.zeros((2 * d_in, d_in), dtype=np.float32)
    X[np.arange(2 * d_in), np.arange(2 * d_in) % d_in] = 1.0 + rng.integers(0, 8, size=2 * d_in) / 8.0
    halves = np.arange(-1, 14) + 0.5                     # -0.5 .. 13.5, each a tie under scale 1
    W = rng.choice(halves, size=(d_out, d_in)).astype(np.float32)
    # every group of 16 spans [-1, 14]: asymmetric scale 1 and zero 1, symmetric scale 2,
    # both exact in fp32, so only the rounding rule decides the ties
    W[:, 0::16], W[:, 1::16] = -1.0, 14.0
    Xb, Wb = synth.f32_to_bf16_bits(X), synth.f32_to_bf16_bits(W)
    assert np.array_equal(synth.bf16_bits_to_f32(Wb), W)
    for group, sym in [(-1, False), (16, False), (-1, True)]:
        sp = dataclasses.replace(spec, group_size=group, sym=sym)
        g = parity.run_gpu(sp, [Wb], [Xb])
        H, _ = R.ref_accumulate_hessian(Xb, "bf16")
        prep = R.ref_prepare_hinv(H, sp.damp, sp.act_order)
        ref = R.ref_quantize_layer(Wb, "bf16", prep, sp.bits, group, sym=sym)
        assert np.array_equal(g["codes"][0], ref["codes"]), (group, sym)
        assert np.array_equal(g["zeros"][0], ref["zeros"]), (group, sym)
        n_ties = int(np.sum(np.abs(ref["grid"].pre - np.floor(ref["grid"].pre) - 0.5) == 0))
        print("exact ties", group, sym, n_ties, flush=True)
        if not sym:
            assert n_ties > d_out * d_in // 4


def test_chunked_accumulation_and_empty_chunk():
    spec = synth.scaled("attn_proj", d_out=64, d_in=256, n_tokens=3000, seq_len=1000)
    announce("chunked accumulation 3000 tokens in 7 chunks")
    import torch
    from post_weight_quantization_03_amd import gptq
    Ws, Xs = parity.make_inputs(spec)
    X = parity.to_torch(Xs[0], "bf16")
    H, key, n = gptq.new_hessian(256)
    for a, b in [(0, 1), (1, 33), (33, 100), (100, 100), (100, 2047), (2047, 2999), (2999, 3000)]:
        gptq.accumulate_hessian(X[a:b], H, key, n)
    torch.cuda.synchronize()
    Href, _ = R.ref_accumulate_hessian(Xs[0], "bf16")
    Hg = H.cpu().numpy().astype(np.float64)
    assert np.linalg.norm(Hg - Href) / np.linalg.norm(Href) <= parity.TOL_H
    assert np.array_equal(Hg, Hg.T)
    assert int(n.item()) == 3000
    np.testing.assert_allclose(key.cpu().numpy(), np.diag(Href), rtol=parity.TOL_KEY)


def test_dead_inputs():
    spec = synth.scaled("attn_proj", d_out=48, d_in=256, n_tokens=1000, seq_len=1000)
    announce("dead inputs")
    Ws, Xs = parity.make_inputs(spec)
    X = Xs[0].copy()
    X[:, [0, 5, 130, 255]] = 0           # four inputs never active
    g = parity.run_gpu(spec, Ws, [X])
    assert g["dead"][0].nonzero()[0].tolist() == [0, 5, 130, 255]
    parity.check_problem(spec, Ws[0], X, g, 0)


def test_degenerate_weight_rows():
    # rows the grid fit must survive: all zero (scale floored at 1e-8, every code at the zero
    # point), constant positive and negative rows (every value on a grid end), values far
    # below the scale floor, and one huge outlier in an otherwise small row
    spec = synth.scaled("attn_proj", d_out=24, d_in=256, n_tokens=1200, seq_len=600)
    announce("degenerate weight rows")
    Ws, Xs = parity.make_inputs(spec)
    Wf = R.widen(Ws[0], spec.dtype).astype(np.float32)
    Wf[0] = 0.0
    Wf[1] = 0.25
    Wf[2] = -0.3
    Wf[3] = 1e-12 * np.sign(Wf[3])
    Wf[4, 17] = 40.0
    Wb = synth.f32_to_bf16_bits(Wf)
    g = parity.run_gpu(spec, [Wb], Xs)
    parity.check_problem(spec, Wb, Xs[0], g, 0)
    zeros, codes = g["zeros"][0], g["codes"][0]
    assert np.all(codes[0] == zeros[:, 0][g["g_idx"][0]])          # the zero row: every code at its zero point
    assert np.all(g["scales"][0][:, 0] == np.float32(1e-8))


def test_not_spd_is_reported():
    announce("not SPD: damp 0, fewer tokens than inputs")
    import torch
    from post_weight_quantization_03_amd import gptq
    spec = synth.scaled("attn_proj", d_out=8, d_in=256, n_tokens=64, seq_len=64)
    Ws, Xs = parity.make_inputs(spec)
    H, key, n = gptq.new_hessian(256)
    gptq.accumulate_hessian(parity.to_torch(Xs[0], "bf16"), H, key, n)
    with pytest.raises(R.NotSPD):
        R.ref_prepare_hinv(R.ref_accumulate_hessian(Xs[0], "bf16")[0], 0.0, True)
    with pytest.raises(gptq.NotSPDError):
        gptq.prepare_hinv(H, key, gptq.Params(damp=0.0, act_order=True))
    torch.cuda.synchronize()


def test_pack_matches_oracle_bit_exactly():
    announce("pack on seeded codes")
    import torch
    from post_weight_quantization_03_amd import gptq
    rng = np.random.default_rng(123)
    for batch, d_out, d_in, ng in [(1, 64, 256, 2), (3, 40, 384, 3), (1, 4096, 512, 4), (2, 8, 8, 1)]:
        codes = rng.integers(0, 16, size=(batch, d_out, d_in)).astype(np.uint8)
        zeros = rng.integers(0, 16, size=(batch, ng, d_out)).astype(np.uint8)
        scales = (rng.random((batch, ng, d_out)) * 0.01).astype(np.float32)
        qw, qz, sf = gptq.pack_int4(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                                    torch.from_numpy(zeros).cuda())
        torch.cuda.synchronize()
        for e in range(batch):
            rq, rz, rs = R.ref_pack_int4(codes[e], scales[e], zeros[e])
            assert np.array_equal(qw[e].cpu().numpy(), rq)
            assert np.array_equal(qz[e].cpu().numpy(), rz)
            assert np.array_equal(sf[e].cpu().numpy().view(np.uint16), rs.view(np.uint16))


def test_deterministic_repeat():
    spec = synth.scaled("attn_proj", d_out=128, d_in=512, n_tokens=4096, seq_len=1024)
    announce("determinism")
    Ws, Xs = parity.make_inputs(spec)
    a = parity.run_gpu(spec, Ws, Xs)
    b = parity.run_gpu(spec, Ws, Xs)
    for k in ("H", "diag_key", "U", "perm", "codes", "scales", "zeros", "g_idx"):
        assert np.array_equal(a[k], b[k]), k
