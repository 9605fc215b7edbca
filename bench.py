"""GPTQ layer-quantization benchmark on one MI355X.

One step = the whole hot path on one layer with its calibration tokens already resident
in HBM: zero the accumulators, H += 2 X^T X over all tokens, dead inputs / ActOrder /
damping / U, the blocked column sweep with lazy updates, and int4 packing.

Default workload: the Llama-8B-shaped attention projection (W 4096 x 4096 bf16,
131072 calibration tokens = 64 sequences x 2048, g128, ActOrder).  Prints ONE JSON line
(metric, value = weights quantized per second, stage times, roofline of the dominant
kernel, CPU-oracle baseline).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "GPTQ layer quantize ms & Gweights/s; SYRK+trailing GEMM % MFMA peak"
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3      # MI355X fp32 (vector with packed math, and matrix)
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="attn_proj")
    ap.add_argument("--chunk", type=int, default=0, help="tokens per accumulate call (0 = all at once)")
    ap.add_argument("--bits", type=int, default=0, help="override the workload's bit width (e.g. 3 for moe)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=32768,
                    help="calibration tokens the CPU oracle processes (its Hessian time is scaled up)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="before warmup, run one plain device copy of this many bytes (counter calibration)")
    return ap.parse_args()


SYRK_SOURCE = os.path.join(ROOT, "post_weight_quantization_03_amd", "csrc", "hessian.hip")


def syrk_traffic(workload: str):
    """HBM bytes per SYRK launch from the committed counter summary of this workload, or None
    when there is none or the SYRK source has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"syrk_mfma_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            k, sep, v = line.partition(":")
            if sep:
                fields[k.strip()] = v.strip()
    with open(SYRK_SOURCE, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    if fields.get("hessian.hip sha256") != digest or "traffic bytes per launch" not in fields:
        return None
    return int(float(fields["traffic bytes per launch"]))


def describe(spec) -> str:
    grid = "per-row" if spec.group_size == -1 else f"g{spec.group_size}"
    lead = f"{spec.batch}x " if spec.batch > 1 else ""
    return (f"{spec.name}: {lead}W {spec.d_out}x{spec.d_in} {spec.dtype}, {spec.n_tokens} tokens, "
            f"{spec.bits}-bit {grid}, block {spec.block_size}, damp {spec.damp}, "
            f"act_order {'on' if spec.act_order else 'off'}")


def cpu_baseline(spec, Ws, Xs, sample_tokens: int):
    """The fp64 oracle on this host: one layer with a bounded token sample; the Hessian
    time is scaled to the full token count (its cost is linear in tokens)."""
    from oracle import gptq_ref as R
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    ns = min(sample_tokens, spec.n_tokens)
    t = {}
    t0 = time.perf_counter()
    R.ref_gptq_layer(Ws[0], [Xs[0][:ns]], spec.dtype, spec.bits, spec.group_size, spec.block_size, spec.damp,
                     spec.act_order, timings=t)
    wall = time.perf_counter() - t0
    full = t["hessian"] * spec.n_tokens / max(ns, 1) + t["prepare"] + t["quantize"]
    weights = spec.d_out * spec.d_in
    return dict(value=weights / full / 1e9, unit="Gweights/s", cores=int(cores), kind="oracle",
                sample=(f"one layer ({spec.d_out}x{spec.d_in}) with {ns} of {spec.n_tokens} tokens; Hessian time "
                        f"scaled x{spec.n_tokens / max(ns, 1):.1f}; measured {wall:.1f} s"),
                ms_per_layer=full * 1e3, stage_s={k: round(v, 3) for k, v in t.items()})


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the layer quantizer runs on a "
              f"single device; multi-GPU sharding is described in the design notes but not built.", file=sys.stderr)
        sys.exit(2)
    import torch
    from post_weight_quantization_03_amd import gptq, synth

    spec = synth.config(args.config)
    if args.bits:
        spec = synth.config(args.config, bits=args.bits)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    Ws = [synth.make_weight(spec, e) for e in range(spec.batch)]
    Xs = [synth.make_activations(spec, e) for e in range(spec.batch)]
    print(f"[bench] generated inputs in {time.perf_counter() - t_gen:.1f} s: {describe(spec)}", file=sys.stderr,
          flush=True)

    def dev_tensor(a):
        if spec.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    batched = spec.batch > 1
    W = torch.stack([dev_tensor(w) for w in Ws]) if batched else dev_tensor(Ws[0])
    X = torch.stack([dev_tensor(x) for x in Xs]) if batched else dev_tensor(Xs[0])
    p = gptq.Params(bits=spec.bits, group_size=spec.group_size, block_size=spec.block_size, damp=spec.damp,
                    act_order=spec.act_order)
    E = spec.batch
    H, key, nseen = gptq.new_hessian(spec.d_in, E if batched else None, dev)
    chunk = args.chunk or spec.n_tokens
    ws_h = torch.empty(gptq.workspace_size(gptq.WS_HESSIAN, E, 0, spec.d_in, chunk, p), dtype=torch.uint8, device=dev)
    ws_p = torch.empty(gptq.workspace_size(gptq.WS_PREPARE, E, 0, spec.d_in, 0, p), dtype=torch.uint8, device=dev)
    ws_q = torch.empty(gptq.workspace_size(gptq.WS_QUANTIZE, E, spec.d_out, spec.d_in, 0, p), dtype=torch.uint8,
                       device=dev)
    stream = torch.cuda.current_stream()
    ev = {k: [] for k in ("hessian", "prepare", "quantize", "pack")}
    if args.copy_bytes:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(record: bool):
        def mark():
            e_ = torch.cuda.Event(enable_timing=True)
            e_.record(stream)
            return e_
        a = mark() if record else None
        H.zero_()
        key.zero_()
        nseen.zero_()
        for t0 in range(0, spec.n_tokens, chunk):
            gptq.accumulate_hessian(X[..., t0:t0 + chunk, :], H, key, nseen, workspace=ws_h)
        b = mark() if record else None
        U, perm, dead = gptq.prepare_hinv(H, key, p, workspace=ws_p)
        c = mark() if record else None
        codes, scales, zeros, g_idx = gptq.quantize_layer(W, U, perm, dead, p, workspace=ws_q)
        d = mark() if record else None
        if spec.d_out % 8 == 0 and spec.bits <= 4:
            gptq.pack_int4(codes, scales, zeros)
        f = mark() if record else None
        if record:
            ev["hessian"].append((a, b))
            ev["prepare"].append((b, c))
            ev["quantize"].append((c, d))
            ev["pack"].append((d, f))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)
    gptq.timing_enable(True)
    gptq.timing_read()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gptq.timing_enable(False)
    syrk_total_ms, syrk_launches = gptq.timing_read()
    ms = wall * 1e3 / args.steps
    stages = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in ev.items()}
    weights = E * spec.d_out * spec.d_in
    value = weights / (ms / 1e3) / 1e9

    # Dominant kernel: the Hessian SYRK.  Algorithmic flops = the lower triangle with its
    # diagonal, 2 * d_in (d_in + 1) / 2 per token and layer; one launch covers one accumulate call.
    launches_per_step = (spec.n_tokens + chunk - 1) // chunk
    syrk_flops = E * spec.d_in * (spec.d_in + 1) * min(chunk, spec.n_tokens)
    syrk_ms = syrk_total_ms / max(syrk_launches, 1)
    achieved = syrk_flops / (syrk_ms / 1e3) / 1e12 if syrk_ms > 0 else 0.0
    mfma = spec.dtype in ("bf16", "f16")
    # fp32 inputs run the vector-ALU SYRK: its peak is the chip's fp32 vector rate
    peak = PEAK_BF16_TFLOPS if mfma else PEAK_F32_TFLOPS
    roof = dict(bound="mfma" if mfma else "alu", kernel="syrk_mfma_kernel" if mfma else "syrk_f32_kernel",
                achieved=round(achieved, 2), peak=peak, unit="TFLOP/s",
                frac=round(achieved / peak, 4), traffic=syrk_traffic(spec.name) if chunk >= spec.n_tokens else None,
                launch_ms=round(syrk_ms, 4), launches=syrk_launches, launches_per_step=launches_per_step,
                flops_per_launch=syrk_flops)
    out = dict(metric=METRIC, value=round(value, 4), unit="Gweights/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=round(ms, 4), higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="bf16->f32", data="synthetic",
               config=dict(workload=describe(spec), d_out=spec.d_out, d_in=spec.d_in, tokens=spec.n_tokens,
                           batch=E, bits=spec.bits, group_size=spec.group_size, act_order=spec.act_order),
               stages_ms={k: round(v, 4) for k, v in stages.items()}, roofline=roof)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(spec, Ws, Xs, args.cpu_sample_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
