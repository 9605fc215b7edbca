"""Seeded synthetic layers and calibration activations for the GPTQ layer quantizer.

This module only draws random numbers and rounds them to the storage dtype; it holds
none of the quantizer's arithmetic.  Both the CPU oracle (``oracle/``) and the HIP
path consume the exact bytes produced here, so parity compares like with like.

Workload recipes.  The calibration sets the pages describe (a few hundred sequences
of 2048 tokens fed through a Llama-style layer, "GPTQ Architecture, in depth",
sections "Groups, act-order and other knobs" and "Worked example: a 7B model") are
stood in for by random activations with the same shapes and the value structure
below; no dataset item is used or reproduced.

* ``W``: i.i.d. N(0, sigma^2), stored as fp32, bf16 or fp16 (round to nearest even
  from fp32).
* ``lognormal`` activations: x[t, c] = N(0, 1) * s_c with s_c = exp(N(0, 1)), so the
  Hessian diagonal spans several decades; optionally a fraction of "outlier"
  channels (chosen without replacement) get s_c multiplied by a factor.
* ``relu2`` activations: x[t, c] = 0 with probability p_zero, else exp(N(0, 1)), i.i.d.
  (positive and sparse, like squared-ReLU MLP inputs).

Random streams (numpy PCG64): W uses ``[seed, 0]``, channel scales ``[seed, 1]``,
token sequence ``s`` uses ``[seed, 2, s]``; every sequence is generated on its own,
so activations can be produced chunk by chunk and in parallel.
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "LayerSpec", "CONFIGS", "config", "scaled", "f32_to_bf16_bits", "bf16_bits_to_f32", "f32_to_f16_bits",
    "make_weight", "make_channel_scales", "make_sequence", "make_activations",
]


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    """One quantization workload: ``batch`` independent layers of shape d_out x d_in."""

    name: str
    d_out: int
    d_in: int
    n_tokens: int              # calibration tokens per layer
    seq_len: int = 2048        # tokens per generated sequence (one RNG stream each)
    dtype: str = "bf16"        # storage dtype of W and X: "bf16", "f16" or "f32"
    w_sigma: float = 0.02
    x_kind: str = "lognormal"  # "lognormal" or "relu2"
    outlier_frac: float = 0.0  # fraction of outlier channels (lognormal only)
    outlier_mult: float = 20.0
    p_zero: float = 0.6        # relu2 only
    bits: int = 4
    group_size: int = 128      # -1 = one grid per row
    block_size: int = 128
    damp: float = 0.01
    act_order: bool = True
    sym: bool = False          # symmetric grid (zero point at the middle level)
    static_groups: bool = False  # groups of consecutive original columns, fitted up front
    batch: int = 1             # independent experts, each with its own seed
    seed: int = 0

    @property
    def weights(self) -> int:
        return self.batch * self.d_out * self.d_in

    def layer_seed(self, e: int) -> int:
        """Seed of expert ``e`` (experts are seeded 100 + e, single layers use ``seed``)."""
        return self.seed + e


CONFIGS = {
    "tiny": LayerSpec("tiny", 256, 256, 2048, dtype="f32", group_size=-1, act_order=False, seed=0),
    "attn_proj": LayerSpec("attn_proj", 4096, 4096, 131072, outlier_frac=0.005, seed=1),
    "mlp_up": LayerSpec("mlp_up", 14336, 4096, 262144, outlier_frac=0.005, act_order=False, seed=2),
    "mlp_down": LayerSpec("mlp_down", 4096, 14336, 262144, w_sigma=0.015, x_kind="relu2", seed=3),
    "moe": LayerSpec("moe", 1408, 2048, 8192, batch=64, seed=100),
}


def config(name: str, **overrides) -> LayerSpec:
    return dataclasses.replace(CONFIGS[name], **overrides)


def scaled(name: str, d_out: int | None = None, d_in: int | None = None,
           n_tokens: int | None = None, batch: int | None = None, **overrides) -> LayerSpec:
    """A smaller instance of a named recipe (same value structure, fewer rows/cols/tokens)."""
    base = CONFIGS[name]
    upd = dict(overrides)
    if d_out is not None:
        upd["d_out"] = d_out
    if d_in is not None:
        upd["d_in"] = d_in
    if n_tokens is not None:
        upd["n_tokens"] = n_tokens
        upd.setdefault("seq_len", min(base.seq_len, n_tokens) if n_tokens > 0 else base.seq_len)
    if batch is not None:
        upd["batch"] = batch
    return dataclasses.replace(base, name=base.name + "_scaled", **upd)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + r) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to fp16 (round-to-nearest-even, numpy's cast) and return the 16-bit patterns."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    if dtype == "f16":
        return f32_to_f16_bits(a32)
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    raise ValueError(dtype)


def make_weight(spec: LayerSpec, e: int = 0) -> np.ndarray:
    """W [d_out, d_in] as fp32, or bf16 / fp16 bit patterns (uint16)."""
    rng = np.random.default_rng([spec.layer_seed(e), 0])
    w = rng.standard_normal((spec.d_out, spec.d_in), dtype=np.float32) * np.float32(spec.w_sigma)
    return _store(w, spec.dtype)


def make_channel_scales(spec: LayerSpec, e: int = 0) -> np.ndarray | None:
    if spec.x_kind != "lognormal":
        return None
    rng = np.random.default_rng([spec.layer_seed(e), 1])
    s = np.exp(rng.standard_normal(spec.d_in)).astype(np.float32)
    n_out = int(round(spec.outlier_frac * spec.d_in))
    if n_out > 0:
        idx = rng.choice(spec.d_in, size=n_out, replace=False)
        s[idx] *= np.float32(spec.outlier_mult)
    return s


def _seq_lengths(spec: LayerSpec) -> list[int]:
    if spec.n_tokens <= 0:
        return []
    full, rem = divmod(spec.n_tokens, spec.seq_len)
    return [spec.seq_len] * full + ([rem] if rem else [])


def make_sequence(spec: LayerSpec, s: int, length: int, scales: np.ndarray | None, e: int = 0) -> np.ndarray:
    """Token-major activations [length, d_in] of sequence ``s`` (storage dtype)."""
    rng = np.random.default_rng([spec.layer_seed(e), 2, s])
    if spec.x_kind == "lognormal":
        x = rng.standard_normal((length, spec.d_in), dtype=np.float32)
        x *= scales[None, :]
    elif spec.x_kind == "relu2":
        keep = rng.random((length, spec.d_in), dtype=np.float32) >= np.float32(spec.p_zero)
        x = np.exp(rng.standard_normal((length, spec.d_in), dtype=np.float32))
        x *= keep
    else:
        raise ValueError(spec.x_kind)
    return _store(x, spec.dtype)


def make_activations(spec: LayerSpec, e: int = 0, out: np.ndarray | None = None,
                     threads: int | None = None) -> np.ndarray:
    """All calibration tokens of layer ``e`` as one token-major array [n_tokens, d_in]."""
    dt = np.uint16 if spec.dtype in ("bf16", "f16") else np.float32
    if out is None:
        out = np.empty((spec.n_tokens, spec.d_in), dtype=dt)
    scales = make_channel_scales(spec, e)
    lens = _seq_lengths(spec)
    starts = np.cumsum([0] + lens[:-1]) if lens else []

    def work(s):
        out[starts[s]:starts[s] + lens[s]] = make_sequence(spec, s, lens[s], scales, e)

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if threads > 1 and len(lens) > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, range(len(lens))))
    else:
        for s in range(len(lens)):
            work(s)
    return out
