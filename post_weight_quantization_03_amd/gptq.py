"""Python binding of libgptq (ctypes): argument marshalling for the C ABI in include/gptq.h.

Every step of the quantizer runs in the HIP library; this module only checks tensor
shapes, dtypes and devices, allocates outputs and workspaces with PyTorch on the current
device, and passes raw pointers and the current HIP stream.  It raises if the shared
library has not been built: there is no fallback path.

Names follow the C ABI: ``accumulate_hessian``, ``prepare_hinv``, ``quantize_layer``,
``pack_int4``.  Tensors may carry a leading batch dimension (independent problems, e.g.
mixture-of-experts layers).
"""

from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgptq.so")
_lib = None

GPTQ_OK, GPTQ_ERR_INVALID_ARG, GPTQ_ERR_NOT_SPD, GPTQ_ERR_HIP, GPTQ_ERR_WORKSPACE, GPTQ_ERR_UNSUPPORTED = 0, -1, -2, -3, -4, -5
GPTQ_ERR_TOO_LARGE = -6
NOALLOC_SCRATCH_BYTES = 64 << 20
WS_HESSIAN, WS_PREPARE, WS_QUANTIZE, WS_W4A16_REPACK, WS_W4A16 = 0, 1, 2, 3, 4

EXPORTED = ("gptq_accumulate_hessian", "gptq_prepare_hinv", "gptq_quantize_layer", "gptq_quantize_layer_noalloc",
            "gptq_accumulate_hessian_grouped", "gptq_pack_int4", "gptq_w4a16_repack", "gptq_w4a16_matmul",
            "gptq_workspace_size", "gptq_status_string", "gptq_version", "gptq_timing_enable", "gptq_timing_read")


class GptqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class NotSPDError(GptqError):
    pass


class _Params(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int), ("group_size", ctypes.c_int), ("block_size", ctypes.c_int),
                ("damp", ctypes.c_float), ("act_order", ctypes.c_int), ("sym", ctypes.c_int),
                ("static_groups", ctypes.c_int)]


@dataclasses.dataclass(frozen=True)
class Params:
    """Quantizer knobs: bits, group_size (-1 = per row), block_size (128), damp, act_order,
    sym (symmetric grid), static_groups (groups of original columns fitted up front)."""

    bits: int = 4
    group_size: int = 128
    block_size: int = 128
    damp: float = 0.01
    act_order: bool = False
    sym: bool = False
    static_groups: bool = False

    def c(self) -> _Params:
        return _Params(self.bits, self.group_size, self.block_size, self.damp, int(self.act_order), int(self.sym),
                       int(self.static_groups))

    def n_groups(self, d_in: int) -> int:
        return 1 if self.group_size == -1 else d_in // self.group_size


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libgptq.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m post_weight_quantization_03_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.gptq_accumulate_hessian.argtypes = [i32, i32, i64, i32, vp, i64, i64, vp, i64, vp, vp, vp, sz, vp]
    L.gptq_accumulate_hessian_grouped.argtypes = [i32, i32, i64, i64, i32, vp, i64, vp, vp, i64, vp, vp, vp, sz, vp]
    L.gptq_prepare_hinv.argtypes = [i32, i32, vp, i64, vp, ctypes.POINTER(_Params), vp, i64, vp, vp, vp, sz, vp]
    L.gptq_quantize_layer.argtypes = [i32, i32, i32, i32, vp, i64, i64, vp, i64, vp, vp, ctypes.POINTER(_Params),
                                      vp, vp, vp, vp, vp, sz, vp]
    L.gptq_quantize_layer_noalloc.argtypes = [i32, i32, i32, i32, vp, i64, i64, vp, i64, vp, vp,
                                              ctypes.POINTER(_Params), vp, vp, vp, vp, vp]
    L.gptq_pack_int4.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    L.gptq_w4a16_repack.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    L.gptq_w4a16_matmul.argtypes = [i32, i32, i32, i32, i32, vp, i64, vp, vp, vp, vp, vp, i64, vp, sz, vp]
    L.gptq_workspace_size.argtypes = [i32, i32, i32, i32, i64, ctypes.POINTER(_Params)]
    L.gptq_workspace_size.restype = sz
    L.gptq_status_string.argtypes = [i32]
    L.gptq_status_string.restype = ctypes.c_char_p
    L.gptq_version.argtypes = []
    L.gptq_version.restype = ctypes.c_char_p
    L.gptq_timing_enable.argtypes = [i32]
    L.gptq_timing_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    for name in ("gptq_accumulate_hessian", "gptq_accumulate_hessian_grouped", "gptq_prepare_hinv", "gptq_quantize_layer", "gptq_quantize_layer_noalloc",
                 "gptq_pack_int4", "gptq_w4a16_repack", "gptq_w4a16_matmul", "gptq_timing_enable",
                 "gptq_timing_read"):
        getattr(L, name).restype = i32
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().gptq_status_string(status).decode()


def _check(status: int, what: str):
    if status == GPTQ_ERR_NOT_SPD:
        raise NotSPDError(status, what)
    if status != GPTQ_OK:
        raise GptqError(status, what)


_DT = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _keep_for(stream, *tensors) -> None:
    """Tensors this module allocated (on torch's current stream) and hands to kernels on
    another stream: tell the caching allocator about that stream, so that their memory
    is not given to new work before the kernels queued there are done with it."""
    if stream is None or stream == torch.cuda.current_stream(stream.device):
        return
    for t in tensors:
        t.record_stream(stream)


def _batched(t: torch.Tensor, nd: int) -> torch.Tensor:
    return t.unsqueeze(0) if t.dim() == nd else t


def workspace_size(which: int, batch: int, d_out: int, d_in: int, n_tokens_hint: int = 0,
                   params: Params | None = None) -> int:
    p = (params or Params()).c()
    return int(lib().gptq_workspace_size(which, batch, d_out, d_in, n_tokens_hint, ctypes.byref(p)))


def _workspace(nbytes: int, device, workspace: torch.Tensor | None, stream=None) -> torch.Tensor:
    if workspace is not None and workspace.numel() >= nbytes:
        return workspace
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    _keep_for(stream, ws)
    return ws


def new_hessian(d_in: int, batch: int | None = None, device="cuda"):
    """Zeroed (H fp32, diag_key fp64, n_seen int64) accumulators."""
    shp = () if batch is None else (batch,)
    return (torch.zeros(*shp, d_in, d_in, dtype=torch.float32, device=device),
            torch.zeros(*shp, d_in, dtype=torch.float64, device=device),
            torch.zeros(*(shp or (1,)), dtype=torch.int64, device=device))


def accumulate_hessian(X: torch.Tensor, H: torch.Tensor, diag_key: torch.Tensor, n_seen: torch.Tensor,
                       workspace: torch.Tensor | None = None, stream=None) -> None:
    """H += 2 X^T X, diag_key += 2 sum x^2 (fp64), n_seen += n for token-major X [(batch,) n, d_in]."""
    Xb = _batched(X, 2)
    Hb = _batched(H, 2)
    batch, n, d_in = Xb.shape
    if X.dtype not in _DT or H.dtype != torch.float32 or diag_key.dtype != torch.float64 or n_seen.dtype != torch.int64:
        raise TypeError("X must be fp32/bf16/fp16, H fp32, diag_key fp64, n_seen int64")
    if Hb.shape != (batch, d_in, d_in) or diag_key.numel() != batch * d_in or n_seen.numel() < batch:
        raise ValueError("shape mismatch between X, H, diag_key, n_seen")
    if Xb.stride(2) != 1 or not Hb.is_contiguous() or not diag_key.is_contiguous():
        raise ValueError("X rows must be contiguous; H and diag_key contiguous")
    ws = _workspace(workspace_size(WS_HESSIAN, batch, 0, d_in, n), X.device, workspace, stream)
    _check(lib().gptq_accumulate_hessian(batch, d_in, n, _DT[X.dtype], Xb.data_ptr(), Xb.stride(1),
                                         Xb.stride(0) if batch > 1 else n * Xb.stride(1), Hb.data_ptr(),
                                         d_in * d_in, diag_key.data_ptr(), n_seen.data_ptr(), ws.data_ptr(),
                                         ws.numel(), _stream(stream)), "gptq_accumulate_hessian")


def accumulate_hessian_grouped(X: torch.Tensor, token_offsets: torch.Tensor, H: torch.Tensor, diag_key: torch.Tensor,
                               n_seen: torch.Tensor, max_tokens: int, workspace: torch.Tensor | None = None,
                               stream=None) -> None:
    """Per-problem token ranges of one buffer: problem e accumulates rows token_offsets[e] ..
    token_offsets[e + 1] - 1 of token-major X [total, d_in] (at most ``max_tokens`` rows each,
    the largest count the caller expects); n_seen[e] += the rows it took."""
    total, d_in = X.shape
    batch = token_offsets.numel() - 1
    Hb = _batched(H, 2)
    if X.dtype not in _DT or H.dtype != torch.float32 or diag_key.dtype != torch.float64 or n_seen.dtype != torch.int64:
        raise TypeError("X must be fp32/bf16/fp16, H fp32, diag_key fp64, n_seen int64")
    if token_offsets.dtype != torch.int64 or not token_offsets.is_contiguous() or batch < 1:
        raise ValueError("token_offsets must be contiguous int64 [batch + 1]")
    if Hb.shape != (batch, d_in, d_in) or diag_key.numel() != batch * d_in or n_seen.numel() < batch:
        raise ValueError("shape mismatch between token_offsets, H, diag_key, n_seen")
    if X.stride(1) != 1 or not Hb.is_contiguous() or not diag_key.is_contiguous():
        raise ValueError("X rows must be contiguous; H and diag_key contiguous")
    ws = _workspace(workspace_size(WS_HESSIAN, batch, 0, d_in, max_tokens), X.device, workspace, stream)
    _check(lib().gptq_accumulate_hessian_grouped(batch, d_in, total, max_tokens, _DT[X.dtype], X.data_ptr(),
                                                 X.stride(0), token_offsets.data_ptr(), Hb.data_ptr(), d_in * d_in,
                                                 diag_key.data_ptr(), n_seen.data_ptr(), ws.data_ptr(), ws.numel(),
                                                 _stream(stream)), "gptq_accumulate_hessian_grouped")


class HessianHook:
    """Calibration hook on a ``torch.nn.Linear`` ("GPTQ Architecture, in depth", "The
    algorithm in code": a hook records each linear layer's inputs batch by batch): every
    forward call adds its input, flattened to token-major [tokens, in_features], to H,
    diag_key and n_seen on the stream the forward runs on.  ``remove()`` detaches it.

    H holds the unnormalised 2 sum x x^T (the running mean of the pages differs by 1/n, and
    the quantizer's results do not depend on that scale); one H serves every weight that
    reads the same input (e.g. the q, k and v projections)."""

    def __init__(self, module: torch.nn.Module, in_features: int | None = None, device=None):
        d_in = in_features if in_features is not None else module.in_features
        dev = device if device is not None else next(module.parameters()).device
        self.H, self.diag_key, self.n_seen = new_hessian(d_in, None, dev)
        self._handle = module.register_forward_pre_hook(self._hook)

    def _hook(self, module, args):
        x = args[0]
        accumulate_hessian(x.reshape(-1, x.shape[-1]), self.H, self.diag_key, self.n_seen)

    def remove(self) -> None:
        self._handle.remove()


def prepare_hinv(H: torch.Tensor, diag_key: torch.Tensor, params: Params, workspace: torch.Tensor | None = None,
                 stream=None):
    """-> (U fp32 [(batch,) d_in, d_in], perm int32 [(batch,) d_in], dead uint8 [(batch,) d_in]).
    Raises NotSPDError if the damped Hessian has no Cholesky factor."""
    Hb = _batched(H, 2)
    batch, d_in, _ = Hb.shape
    if not Hb.is_contiguous() or not diag_key.is_contiguous():
        raise ValueError("H and diag_key must be contiguous")
    shp = H.shape[:-1]
    U = torch.empty(*H.shape, dtype=torch.float32, device=H.device)
    perm = torch.empty(*shp, dtype=torch.int32, device=H.device)
    dead = torch.empty(*shp, dtype=torch.uint8, device=H.device)
    _keep_for(stream, U, perm, dead)
    ws = _workspace(workspace_size(WS_PREPARE, batch, 0, d_in, 0, params), H.device, workspace, stream)
    p = params.c()
    _check(lib().gptq_prepare_hinv(batch, d_in, Hb.data_ptr(), d_in * d_in, diag_key.data_ptr(), ctypes.byref(p),
                                   U.data_ptr(), d_in * d_in, perm.data_ptr(), dead.data_ptr(), ws.data_ptr(),
                                   ws.numel(), _stream(stream)), "gptq_prepare_hinv")
    return U, perm, dead


def quantize_layer(W: torch.Tensor, U: torch.Tensor, perm: torch.Tensor, dead: torch.Tensor, params: Params,
                   workspace: torch.Tensor | None = None, stream=None):
    """-> (codes uint8 [(b,) d_out, d_in] original order, scales fp32 [(b,) n_groups, d_out],
    zeros uint8 [(b,) n_groups, d_out], g_idx int32 [(b,) d_in])."""
    Wb = _batched(W, 2)
    batch, d_out, d_in = Wb.shape
    if W.dtype not in _DT:
        raise TypeError("W must be fp32/bf16/fp16")
    if Wb.stride(2) != 1 or not U.is_contiguous() or not perm.is_contiguous() or not dead.is_contiguous():
        raise ValueError("W rows, U, perm and dead must be contiguous")
    ng = params.n_groups(d_in)
    lead = W.shape[:-2]
    codes = torch.empty(*lead, d_out, d_in, dtype=torch.uint8, device=W.device)
    scales = torch.empty(*lead, ng, d_out, dtype=torch.float32, device=W.device)
    zeros = torch.empty(*lead, ng, d_out, dtype=torch.uint8, device=W.device)
    g_idx = torch.empty(*lead, d_in, dtype=torch.int32, device=W.device)
    _keep_for(stream, codes, scales, zeros, g_idx)
    ws = _workspace(workspace_size(WS_QUANTIZE, batch, d_out, d_in, 0, params), W.device, workspace, stream)
    p = params.c()
    _check(lib().gptq_quantize_layer(batch, d_out, d_in, _DT[W.dtype], Wb.data_ptr(), Wb.stride(1),
                                     Wb.stride(0) if batch > 1 else d_out * Wb.stride(1), U.data_ptr(),
                                     d_in * d_in, perm.data_ptr(), dead.data_ptr(), ctypes.byref(p),
                                     codes.data_ptr(), scales.data_ptr(), zeros.data_ptr(), g_idx.data_ptr(),
                                     ws.data_ptr(), ws.numel(), _stream(stream)), "gptq_quantize_layer")
    return codes, scales, zeros, g_idx


def quantize_layer_noalloc(W: torch.Tensor, U: torch.Tensor, perm: torch.Tensor, dead: torch.Tensor, params: Params,
                           out=None, stream=None):
    """gptq_quantize_layer_noalloc: the same results as :func:`quantize_layer` with the
    library's fixed device scratch instead of a workspace.  ``out`` = (codes, scales,
    zeros, g_idx) preallocated by the caller (shapes as returned by quantize_layer);
    without it they are allocated here, but the C call itself never allocates."""
    Wb = _batched(W, 2)
    batch, d_out, d_in = Wb.shape
    if W.dtype not in _DT:
        raise TypeError("W must be fp32/bf16/fp16")
    if Wb.stride(2) != 1 or not U.is_contiguous() or not perm.is_contiguous() or not dead.is_contiguous():
        raise ValueError("W rows, U, perm and dead must be contiguous")
    ng = params.n_groups(d_in)
    lead = W.shape[:-2]
    if out is None:
        out = (torch.empty(*lead, d_out, d_in, dtype=torch.uint8, device=W.device),
               torch.empty(*lead, ng, d_out, dtype=torch.float32, device=W.device),
               torch.empty(*lead, ng, d_out, dtype=torch.uint8, device=W.device),
               torch.empty(*lead, d_in, dtype=torch.int32, device=W.device))
        _keep_for(stream, *out)
    codes, scales, zeros, g_idx = out
    want = [((*lead, d_out, d_in), torch.uint8), ((*lead, ng, d_out), torch.float32),
            ((*lead, ng, d_out), torch.uint8), ((*lead, d_in), torch.int32)]
    for t, (shape, dt) in zip(out, want):
        if tuple(t.shape) != tuple(shape) or t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"output tensor must be contiguous {dt} of shape {shape}")
    p = params.c()
    _check(lib().gptq_quantize_layer_noalloc(batch, d_out, d_in, _DT[W.dtype], Wb.data_ptr(), Wb.stride(1),
                                             Wb.stride(0) if batch > 1 else d_out * Wb.stride(1), U.data_ptr(),
                                             d_in * d_in, perm.data_ptr(), dead.data_ptr(), ctypes.byref(p),
                                             codes.data_ptr(), scales.data_ptr(), zeros.data_ptr(), g_idx.data_ptr(),
                                             _stream(stream)), "gptq_quantize_layer_noalloc")
    return codes, scales, zeros, g_idx


def pack_int4(codes: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor, stream=None):
    """-> (qweight int32 [(b,) d_in/8, d_out], qzeros int32 [(b,) n_groups, d_out/8],
    scales fp16 [(b,) n_groups, d_out])."""
    cb = _batched(codes, 2)
    batch, d_out, d_in = cb.shape
    ng = scales.shape[-2]
    if not (codes.is_contiguous() and scales.is_contiguous() and zeros.is_contiguous()):
        raise ValueError("codes, scales and zeros must be contiguous")
    lead = codes.shape[:-2]
    qweight = torch.empty(*lead, d_in // 8, d_out, dtype=torch.int32, device=codes.device)
    qzeros = torch.empty(*lead, ng, d_out // 8, dtype=torch.int32, device=codes.device)
    sf16 = torch.empty(*lead, ng, d_out, dtype=torch.float16, device=codes.device)
    _keep_for(stream, qweight, qzeros, sf16)
    _check(lib().gptq_pack_int4(batch, d_out, d_in, ng, codes.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
                                qweight.data_ptr(), qzeros.data_ptr(), sf16.data_ptr(), _stream(stream)),
           "gptq_pack_int4")
    return qweight, qzeros, sf16


TIME_SYRK, TIME_LAZY_GEMM, TIME_SWEEP, TIME_PACK, TIME_W4A16 = 0, 1, 2, 3, 4


def w4a16_repack(qweight: torch.Tensor, g_idx: torch.Tensor, n_groups: int, workspace: torch.Tensor | None = None,
                 stream=None):
    """Serving layout of a packed layer: (qweight_s int32 [(b,) d_in/8, d_out], order int32
    [(b,) d_in]) with the inputs sorted by group.  Raises GptqError on a malformed g_idx."""
    qb = _batched(qweight, 2)
    batch, rows8, d_out = qb.shape
    d_in = rows8 * 8
    if qweight.dtype != torch.int32 or g_idx.dtype != torch.int32 or g_idx.numel() != batch * d_in:
        raise TypeError("qweight and g_idx must be int32, g_idx [(b,) d_in]")
    if not qweight.is_contiguous() or not g_idx.is_contiguous():
        raise ValueError("qweight and g_idx must be contiguous")
    qs = torch.empty_like(qweight)
    order = torch.empty_like(g_idx)
    _keep_for(stream, qs, order)
    ws = _workspace(workspace_size(WS_W4A16_REPACK, batch, d_out, d_in), qweight.device, workspace, stream)
    _check(lib().gptq_w4a16_repack(batch, d_out, d_in, n_groups, qweight.data_ptr(), g_idx.data_ptr(), qs.data_ptr(),
                                   order.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream)), "gptq_w4a16_repack")
    return qs, order


def w4a16_matmul(X: torch.Tensor, qweight_s: torch.Tensor, qzeros: torch.Tensor, scales_f16: torch.Tensor,
                 order: torch.Tensor | None = None, out: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y fp32 [m, d_out] = X What^T from the packed tensors (X [m, d_in] bf16 / fp16).
    ``order`` from :func:`w4a16_repack`, or None when qweight is in input order with
    contiguous groups."""
    m, d_in = X.shape
    d_out = qweight_s.shape[-1]
    n_groups = scales_f16.shape[0]
    if X.dtype not in (torch.bfloat16, torch.float16) or X.stride(1) != 1:
        raise TypeError("X must be bf16 or fp16 with contiguous rows")
    if qweight_s.dtype != torch.int32 or qzeros.dtype != torch.int32 or scales_f16.dtype != torch.float16:
        raise TypeError("qweight and qzeros int32, scales fp16")
    if not (qweight_s.is_contiguous() and qzeros.is_contiguous() and scales_f16.is_contiguous()):
        raise ValueError("packed tensors must be contiguous")
    if order is not None and (order.dtype != torch.int32 or order.numel() != d_in or not order.is_contiguous()):
        raise ValueError("order must be contiguous int32 [d_in]")
    Y = out if out is not None else torch.empty(m, d_out, dtype=torch.float32, device=X.device)
    if out is None:
        _keep_for(stream, Y)
    gsz = -1 if n_groups == 1 else d_in // n_groups
    ws = _workspace(workspace_size(WS_W4A16, 1, d_out, d_in, m, Params(group_size=gsz)), X.device, workspace, stream)
    _check(lib().gptq_w4a16_matmul(m, d_out, d_in, n_groups, _DT[X.dtype], X.data_ptr(), X.stride(0),
                                   qweight_s.data_ptr(), None if order is None else order.data_ptr(), qzeros.data_ptr(),
                                   scales_f16.data_ptr(), Y.data_ptr(), Y.stride(0), ws.data_ptr(), ws.numel(),
                                   _stream(stream)), "gptq_w4a16_matmul")
    return Y


def timing_enable(on: bool = True, kinds=None) -> None:
    """Start/stop recording HIP events around the launches of the timed kernel classes
    (``kinds``: an iterable of TIME_* values, all of them when None)."""
    mask = 0
    if on:
        mask = -1 if kinds is None else sum(1 << k for k in set(kinds))
    _check(lib().gptq_timing_enable(mask), "gptq_timing_enable")


def timing_read(which: int = TIME_SYRK):
    """(summed kernel milliseconds, launches) of one timed class since its previous read."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    _check(lib().gptq_timing_read(which, ctypes.byref(ms), ctypes.byref(n)), "gptq_timing_read")
    return ms.value, n.value


def gptq_layer(W: torch.Tensor, X_chunks, params: Params, stream=None):
    """Whole layer: accumulate H over the chunks, prepare U, quantize.  Returns a dict."""
    lead = W.shape[:-2]
    d_in = W.shape[-1]
    H, key, n = new_hessian(d_in, lead[0] if lead else None, W.device)
    for Xc in X_chunks:
        accumulate_hessian(Xc, H, key, n, stream=stream)
    U, perm, dead = prepare_hinv(H, key, params, stream=stream)
    codes, scales, zeros, g_idx = quantize_layer(W, U, perm, dead, params, stream=stream)
    return dict(H=H, diag_key=key, n_seen=n, U=U, perm=perm, dead=dead, codes=codes, scales=scales,
                zeros=zeros, g_idx=g_idx)
