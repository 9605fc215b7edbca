"""The allocation-free quantize entry point against the workspace one, through the C ABI.

gptq_quantize_layer_noalloc takes no workspace: its scratch lives in a fixed device array
of the library.  Two calls in a row (the second on a smaller problem, so the array holds
the first call's leftovers) must give the same codes, scales, zeros and g_idx as
gptq_quantize_layer with a caller workspace, bit for bit: both run the same kernels on
the same inputs.  A problem above the array's size is rejected before any launch.
"""
import ctypes

import numpy as np
import pytest

from post_weight_quantization_03_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu


def _prepared(spec):
    import torch
    from post_weight_quantization_03_amd import gptq
    Ws, Xs = parity.make_inputs(spec)
    p = parity.params_of(spec)
    batched = spec.batch > 1
    W = torch.stack([parity.to_torch(w, spec.dtype) for w in Ws]) if batched else parity.to_torch(Ws[0], spec.dtype)
    X = torch.stack([parity.to_torch(x, spec.dtype) for x in Xs]) if batched else parity.to_torch(Xs[0], spec.dtype)
    H, key, n = gptq.new_hessian(spec.d_in, spec.batch if batched else None)
    gptq.accumulate_hessian(X, H, key, n)
    U, perm, dead = gptq.prepare_hinv(H, key, p)
    return W, U, perm, dead, p


def _noalloc(W, U, perm, dead, p):
    """Outputs allocated here (by the caller); the entry point itself allocates nothing."""
    import torch
    from post_weight_quantization_03_amd import gptq
    Wb = W if W.dim() == 3 else W.unsqueeze(0)
    batch, d_out, d_in = Wb.shape
    ng = p.n_groups(d_in)
    codes = torch.full((batch, d_out, d_in), 255, dtype=torch.uint8, device=W.device)
    scales = torch.full((batch, ng, d_out), -1.0, dtype=torch.float32, device=W.device)
    zeros = torch.full((batch, ng, d_out), 255, dtype=torch.uint8, device=W.device)
    g_idx = torch.full((batch, d_in), -1, dtype=torch.int32, device=W.device)
    pc = p.c()
    st = gptq.lib().gptq_quantize_layer_noalloc(
        batch, d_out, d_in, gptq._DT[W.dtype], Wb.data_ptr(), Wb.stride(1), Wb.stride(0), U.data_ptr(), d_in * d_in,
        perm.data_ptr(), dead.data_ptr(), ctypes.byref(pc), codes.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
        g_idx.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == gptq.GPTQ_OK, gptq.status_string(st)
    return codes, scales, zeros, g_idx


def test_noalloc_matches_workspace_entry_point_twice():
    import torch
    from post_weight_quantization_03_amd import gptq
    big = synth.scaled("moe", d_out=352, d_in=1024, n_tokens=2500, batch=3, seq_len=500)     # 1.08M weights
    small = synth.scaled("attn_proj", d_out=72, d_in=384, n_tokens=1500, seq_len=500, group_size=64)
    for spec in (big, small):
        print(f"\n[gpu-case] no-alloc quantize vs workspace quantize: {spec}", flush=True)
        W, U, perm, dead, p = _prepared(spec)
        ref = gptq.quantize_layer(W, U, perm, dead, p)
        got = _noalloc(W, U, perm, dead, p)
        torch.cuda.synchronize()
        for name, a, b in zip(("codes", "scales", "zeros", "g_idx"), ref, got):
            a = a.cpu().numpy().reshape(b.shape)
            assert np.array_equal(a, b.cpu().numpy()), name


def test_noalloc_rejects_problems_above_its_scratch():
    import torch
    from post_weight_quantization_03_amd import gptq
    L = gptq.lib()
    pc = gptq.Params().c()
    # 8192 x 8192 weights need 9 bytes each: far above the fixed scratch; rejected before
    # any pointer is touched (all pointers are dummies)
    st = L.gptq_quantize_layer_noalloc(1, 8192, 8192, 1, 16, 8192, 0, 16, 8192 * 8192, 16, 16, ctypes.byref(pc),
                                       16, 16, 16, 16, None)
    assert st == gptq.GPTQ_ERR_TOO_LARGE
    torch.cuda.synchronize()
