"""GPTQ layer-quantization benchmark on one MI355X.

One step = the whole hot path on one layer with its calibration tokens already resident
in HBM: zero the accumulators, H += 2 X^T X over all tokens, dead inputs / ActOrder /
damping / U, the blocked column sweep with lazy updates, and int4 packing.

Default workload: the widest single-GPU configuration, the MLP down projection (W 4096 x
14336 bf16, 262144 calibration tokens = 128 sequences x 2048 from ReLU^2-like sparse
activations, g128, ActOrder, packed).  Prints ONE JSON line: metric, value = weights
quantized per second, stage times, the roofline of the dominant kernel (the Hessian SYRK)
and of the lazy-update products, the column sweep and the packing, and the CPU-oracle
baseline.
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
BLOCK = 128


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="mlp_down")
    ap.add_argument("--chunk", type=int, default=0, help="tokens per accumulate call (0 = all at once)")
    ap.add_argument("--bits", type=int, default=0, help="override the workload's bit width (e.g. 3 for moe)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-serve", action="store_true", help="skip the W4A16 decode measurement")
    ap.add_argument("--cpu-sample-tokens", type=int, default=2048,
                    help="calibration tokens the CPU oracle processes (its Hessian time is scaled up)")
    ap.add_argument("--cpu-sample-rows", type=int, default=64,
                    help="weight rows the CPU oracle sweeps (its sweep time is scaled up; rows are independent)")
    ap.add_argument("--cpu-sample-dim", type=int, default=4096,
                    help="leading input channels of the CPU oracle's factorization and sweep (times scaled up)")
    ap.add_argument("--kernel-timing", choices=("all", "syrk"), default="syrk",
                    help="kernel classes bracketed by HIP events inside the timed steps; with 'syrk' the "
                         "other classes are timed over as many extra instrumented steps afterwards")
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


def lazy_products(d_out: int, d_in: int, batch: int):
    """(M, N, K) of every lazy-update product of one layer, in the order the library issues
    them: after the left half of a block range is swept, its errors reach the right half in
    one product (the same recursion as the library's host code)."""
    out = []

    def rec(b0, b1):
        if b1 - b0 == 1:
            return
        bm = b0 + (b1 - b0) // 2
        rec(b0, bm)
        out.append((d_out, (b1 - bm) * BLOCK, (bm - b0) * BLOCK))
        rec(bm, b1)

    rec(0, d_in // BLOCK)
    return out


def cpu_baseline(spec, Ws, Xs, sample_tokens: int, sample_rows: int, sample_dim: int):
    """The fp64 oracle on this host, on a bounded sample of one layer, each stage scaled by
    the cost model of the pages ("Same Ruler, Smarter Placement: GPTQ", 1.10: Hessian
    O(d_in^2 n), factorization O(d_in^3), column loop O(d_out d_in^2)): the Hessian of all
    channels over ``sample_tokens`` tokens (x n / tokens); the factorization and the sweep
    of ``sample_rows`` rows on the leading ``sample_dim`` input channels (x (d_in / dim)^3
    and x (d_in / dim)^2 (d_out / rows))."""
    from oracle import gptq_ref as R
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    ns = min(sample_tokens, spec.n_tokens)
    nr = min(sample_rows, spec.d_out)
    dm = min(sample_dim, spec.d_in)
    t0 = time.perf_counter()
    H, _ = R.ref_accumulate_hessian(Xs[0][:ns], spec.dtype)
    t1 = time.perf_counter()
    prep = R.ref_prepare_hinv(H[:dm, :dm], spec.damp, spec.act_order)
    t2 = time.perf_counter()
    R.ref_quantize_layer(np.ascontiguousarray(Ws[0][:nr, :dm]), spec.dtype, prep, spec.bits, spec.group_size,
                         sym=spec.sym, static_groups=spec.static_groups)
    t3 = time.perf_counter()
    t = dict(hessian=t1 - t0, prepare=t2 - t1, quantize=t3 - t2)
    fd = spec.d_in / dm
    scaled = dict(hessian=t["hessian"] * spec.n_tokens / max(ns, 1), prepare=t["prepare"] * fd ** 3,
                  quantize=t["quantize"] * fd ** 2 * spec.d_out / max(nr, 1))
    full = sum(scaled.values())
    weights = spec.d_out * spec.d_in     # one layer (one expert of a batch)
    return dict(value=weights / full / 1e9, unit="Gweights/s", cores=cores, kind="oracle",
                sample=(f"one layer ({spec.d_out}x{spec.d_in}): Hessian of all channels over {ns} of "
                        f"{spec.n_tokens} tokens (x{spec.n_tokens / max(ns, 1):.1f}); factorization and sweep of "
                        f"{nr} rows on the leading {dm} input channels (x{fd ** 3:.1f} and "
                        f"x{fd ** 2 * spec.d_out / max(nr, 1):.1f}, by the O(d^3) and O(d_out d^2) cost model); "
                        f"measured {t3 - t0:.1f} s"),
                blas_threads=blas_threads, ms_per_layer=full * 1e3, stage_s={k: round(v, 3) for k, v in t.items()},
                stage_s_scaled={k: round(v, 2) for k, v in scaled.items()})


def w4a16_decode(gptq, torch, qweight, qzeros, scales_f16, g_idx, n_groups, rows, dtype, reps):
    """Decode-time W4A16 product on the benchmark layer's own checkpoint: repack once, then
    time gptq_w4a16_matmul with ``rows`` activation rows over enough copies of the packed
    weights (rotated) that no copy is still in the 256 MB last-level cache when it is read
    again.  Algorithmic bytes per call: qweight, scales, qzeros, X and Y once."""
    d_in = qweight.shape[-2] * 8
    d_out = qweight.shape[-1]
    qs, order = gptq.w4a16_repack(qweight, g_idx, n_groups)
    per = qs.numel() * 4 + scales_f16.numel() * 2 + qzeros.numel() * 4
    copies = max(2, -(-(768 << 20) // per))
    sets = [(qs.clone(), qzeros.clone(), scales_f16.clone()) for _ in range(copies)]
    X = torch.randn(rows, d_in, device=qs.device).to(dtype)
    Y = torch.empty(rows, d_out, dtype=torch.float32, device=qs.device)
    for q_, z_, s_ in sets[:2]:
        gptq.w4a16_matmul(X, q_, z_, s_, order, out=Y)
    torch.cuda.synchronize()
    gptq.timing_enable(True, [gptq.TIME_W4A16])
    gptq.timing_read(gptq.TIME_W4A16)
    for i in range(reps):
        q_, z_, s_ = sets[i % copies]
        gptq.w4a16_matmul(X, q_, z_, s_, order, out=Y)
    torch.cuda.synchronize()
    gptq.timing_enable(False)
    total, n = gptq.timing_read(gptq.TIME_W4A16)
    call_ms = total / max(n, 1)
    alg = per + rows * d_in * 2 + rows * d_out * 4
    gbs = alg / (call_ms / 1e3) / 1e9 if call_ms > 0 else 0.0
    return dict(bound="hbm", kernel="w4a16_kernel + w4a16_reduce_kernel", rows=rows, achieved=round(gbs, 1),
                peak=PEAK_HBM_GBS, unit="GB/s", frac=round(gbs / PEAK_HBM_GBS, 4), traffic=None,
                launch_ms=round(call_ms, 5), calls=n, bytes_per_call=alg, weight_copies=copies,
                tflops=round(2.0 * rows * d_in * d_out / (call_ms / 1e3) / 1e12, 2) if call_ms > 0 else 0.0)


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
        if spec.dtype == "f16":
            return torch.from_numpy(a.view(np.float16)).to(dev)
        return torch.from_numpy(a).to(dev)

    batched = spec.batch > 1
    W = torch.stack([dev_tensor(w) for w in Ws]) if batched else dev_tensor(Ws[0])
    X = torch.stack([dev_tensor(x) for x in Xs]) if batched else dev_tensor(Xs[0])
    p = gptq.Params(bits=spec.bits, group_size=spec.group_size, block_size=spec.block_size, damp=spec.damp,
                    act_order=spec.act_order, sym=spec.sym, static_groups=spec.static_groups)
    E = spec.batch
    H, key, nseen = gptq.new_hessian(spec.d_in, E if batched else None, dev)
    chunk = args.chunk or spec.n_tokens
    ws_h = torch.empty(gptq.workspace_size(gptq.WS_HESSIAN, E, 0, spec.d_in, chunk, p), dtype=torch.uint8, device=dev)
    ws_p = torch.empty(gptq.workspace_size(gptq.WS_PREPARE, E, 0, spec.d_in, 0, p), dtype=torch.uint8, device=dev)
    ws_q = torch.empty(gptq.workspace_size(gptq.WS_QUANTIZE, E, spec.d_out, spec.d_in, 0, p), dtype=torch.uint8,
                       device=dev)
    stream = torch.cuda.current_stream()
    ev = {k: [] for k in ("hessian", "prepare", "quantize", "pack")}
    packs = spec.d_out % 8 == 0 and spec.bits <= 4
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
        if packs:
            gptq.pack_int4(codes, scales, zeros)
        f = mark() if record else None
        if record:
            ev["hessian"].append((a, b))
            ev["prepare"].append((b, c))
            ev["quantize"].append((c, d))
            ev["pack"].append((d, f))

    kinds = dict(syrk=gptq.TIME_SYRK, lazy=gptq.TIME_LAZY_GEMM, sweep=gptq.TIME_SWEEP, pack=gptq.TIME_PACK)

    def read_kernels():
        return {k: gptq.timing_read(v) for k, v in kinds.items()}

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)
    gptq.timing_enable(True, None if args.kernel_timing == "all" else [gptq.TIME_SYRK])
    read_kernels()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gptq.timing_enable(False)
    kt = read_kernels()
    timing_note = "all timed kernel classes bracketed by HIP events inside the timed steps"
    if args.kernel_timing == "syrk":
        # only the SYRK counts from the timed steps; the other classes from as many extra steps
        gptq.timing_enable(True, [gptq.TIME_LAZY_GEMM, gptq.TIME_SWEEP, gptq.TIME_PACK])
        for _ in range(args.steps):
            step(False)
        torch.cuda.synchronize()
        gptq.timing_enable(False)
        extra = read_kernels()
        for k in ("lazy", "sweep", "pack"):
            kt[k] = extra[k]
        timing_note = "SYRK events inside the timed steps; the other classes over as many instrumented steps after them"
    ms = wall * 1e3 / args.steps
    stages = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in ev.items()}
    weights = E * spec.d_out * spec.d_in
    value = weights / (ms / 1e3) / 1e9

    # Dominant kernel: the Hessian SYRK.  Algorithmic flops = the lower triangle with its
    # diagonal, 2 * d_in (d_in + 1) / 2 per token and layer; one launch covers one accumulate call.
    launches_per_step = (spec.n_tokens + chunk - 1) // chunk
    syrk_flops = E * spec.d_in * (spec.d_in + 1) * min(chunk, spec.n_tokens)
    syrk_total_ms, syrk_launches = kt["syrk"]
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

    # Lazy trailing updates: d_out d_in (d_in - 128) algorithmic flops per layer (every pair of
    # columns in different 128-blocks meets once), over the summed time of all their products;
    # beside it their operand bytes (A, B read once, C read and written) as an HBM rate.
    prods = lazy_products(spec.d_out, spec.d_in, E)
    lazy_flops = E * spec.d_out * spec.d_in * (spec.d_in - BLOCK)
    lazy_bytes = E * sum(4 * (m * k + k * n + 2 * m * n) for m, n, k in prods)
    lazy_total, lazy_n = kt["lazy"]
    lazy_step_ms = lazy_total / max(args.steps, 1)
    lazy_tf = lazy_flops / (lazy_step_ms / 1e3) / 1e12 if lazy_step_ms > 0 else 0.0
    lazy_gbs = lazy_bytes / (lazy_step_ms / 1e3) / 1e9 if lazy_step_ms > 0 else 0.0
    roof_lazy = dict(bound="mfma", kernel="gemm_x6_kernel / gemm_f32_kernel (lazy-update instantiations)",
                     achieved=round(lazy_tf, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                     frac=round(lazy_tf / PEAK_BF16_TFLOPS, 4), traffic=None,
                     ms_per_step=round(lazy_step_ms, 4), launches=lazy_n, launches_per_step=len(prods),
                     flops_per_step=lazy_flops, hbm_bytes_per_step=lazy_bytes, hbm_achieved_gbs=round(lazy_gbs, 1),
                     hbm_frac=round(lazy_gbs / PEAK_HBM_GBS, 4))

    # Column sweep: per 128-column launch it reads the rows' fp32 block columns (4 B), writes
    # their errors (4 B) and codes (1 B), and reads the 128 x 128 fp32 diagonal block of U.
    sweep_bytes = E * (spec.d_out * BLOCK * 9 + BLOCK * BLOCK * 4)
    sw_total, sw_n = kt["sweep"]
    sw_ms = sw_total / max(sw_n, 1)
    sw_gbs = sweep_bytes / (sw_ms / 1e3) / 1e9 if sw_ms > 0 else 0.0
    roof_sweep = dict(bound="hbm", kernel="block_sweep_kernel", achieved=round(sw_gbs, 1), peak=PEAK_HBM_GBS,
                      unit="GB/s", frac=round(sw_gbs / PEAK_HBM_GBS, 4), traffic=None, launch_ms=round(sw_ms, 5),
                      launches=sw_n, launches_per_step=spec.d_in // BLOCK, bytes_per_launch=sweep_bytes)
    out_extra = dict(roofline_lazy_gemm=roof_lazy, roofline_sweep=roof_sweep)
    if packs:
        # packing: codes read (1 B) and qweight written (0.5 B) per weight; per group and row the
        # fp32 scale and u8 zero read, the fp16 scale and half a qzeros byte written
        ng = 1 if spec.group_size == -1 else spec.d_in // spec.group_size
        pack_bytes = E * (spec.d_out * spec.d_in * 3 // 2 + ng * spec.d_out * 15 // 2)
        pk_total, pk_n = kt["pack"]
        pk_ms = pk_total / max(pk_n, 1)
        pk_gbs = pack_bytes / (pk_ms / 1e3) / 1e9 if pk_ms > 0 else 0.0
        out_extra["roofline_pack"] = dict(bound="hbm", kernel="pack_qweight_kernel + pack_meta_kernel",
                                          achieved=round(pk_gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                                          frac=round(pk_gbs / PEAK_HBM_GBS, 4), traffic=None,
                                          launch_ms=round(pk_ms, 5), launches=pk_n, bytes_per_launch=pack_bytes)
    if packs and spec.bits == 4 and spec.batch == 1 and spec.dtype in ("bf16", "f16") and not args.no_serve:
        # the serving product of the layer just quantized: its packed checkpoint from one more step
        U, perm, dead = gptq.prepare_hinv(H, key, p, workspace=ws_p)
        codes, scales, zeros, g_idx = gptq.quantize_layer(W, U, perm, dead, p, workspace=ws_q)
        qw, qz, sf = gptq.pack_int4(codes, scales, zeros)
        ng = scales.shape[-2]
        xdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float16
        out_extra["roofline_w4a16_decode"] = [
            w4a16_decode(gptq, torch, qw, qz, sf, g_idx, ng, rows, xdt, reps=200) for rows in (1, 16)]
        del U, codes, qw, qz, sf
    out = dict(metric=METRIC, value=round(value, 4), unit="Gweights/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=round(ms, 4), higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype=f"{spec.dtype}->f32", data="synthetic",
               config=dict(workload=describe(spec), d_out=spec.d_out, d_in=spec.d_in, tokens=spec.n_tokens,
                           batch=E, bits=spec.bits, group_size=spec.group_size, act_order=spec.act_order),
               stages_ms={k: round(v, 4) for k, v in stages.items()}, roofline=roof, **out_extra,
               kernel_timing=timing_note)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(spec, Ws, Xs, args.cpu_sample_tokens, args.cpu_sample_rows,
                                           args.cpu_sample_dim)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
