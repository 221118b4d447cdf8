"""Benchmark of the fused exact-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the C-ABI forward (the whole hot path: tiling, both
MFMA products, online softmax, epilogue) over one batch of seeded synthetic
inputs already resident in HBM.  The default workload is the causal bf16
B=2 H=16 N=8192 d=128 forward.  Throughput is F / t with F = 4*B*H*N^2*d,
halved when causal.  Prints ONE JSON line with a "roofline" object (achieved
TFLOP/s of the kernel against the dense bf16 MFMA peak, timed with HIP events
on the stream the kernel runs on) and a "cpu_baseline" object (the fp64 oracle
timed on a bounded sample of the same workload's heads on the host cores).

Before the W warm-up steps a settle phase runs back-to-back launches for about
--settle-ms of GPU time (default 300 ms) and is reported under "settle": the
chip's clock settles only after tens of milliseconds of sustained MFMA load,
and launches in the first ~50 ms run up to 20% slower than the steady state
that the K timed steps then measure.  The settle phase is untimed extra
warm-up; W and K keep their exact meaning, and every timed step does the
whole call.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (bf16, causal, N=8192, d=128) and % of MFMA peak"
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3, "fp8": 5033.2}   # MI355X dense, published
PEAK_HBM_GBS = 8000.0                                             # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="back-to-back launches for about this much GPU time before the "
                         "warm-up, so the clock has settled (reported as 'settle')")
    ap.add_argument("--workload", default="bf16_causal_n8192_d128")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tile-cfg", type=int, default=0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run plain device copies of this size (MiB) so that "
                         "HBM byte counters can be scaled against a known transfer")
    return ap.parse_args()


def measured_traffic(w):
    """HBM bytes per call recorded under profiles/ for this workload, or None
    when the kernel source or its build flags changed since the counters were
    taken (the record keeps the fingerprint of every source it covers)."""
    from exact_attention_77_amd.build import fingerprint
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        rec = json.load(open(path))[w.name]
        if any(fingerprint(os.path.basename(src)) != fp for src, fp in rec["fingerprints"].items()):
            return None
    except (OSError, KeyError, ValueError, AttributeError):
        return None
    return rec["read_bytes"] + rec["write_bytes"]


def launch_stats(step, stream, dev, n):
    """After the timed region: n launches with one HIP event pair each (median
    and minimum), then three cold launches, each after a 512 MiB scrub write
    that evicts the inputs from L2 and the 256 MB last-level cache."""
    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    lat = sorted(a.elapsed_time(b) for a, b in ev)
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(3):
        scrub.fill_(i + 1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    del scrub
    return {"launches": n, "median_ms": round(lat[n // 2], 5), "min_ms": round(lat[0], 5),
            "cold_ms": round(sorted(cold)[1], 5), "cold_scrub_bytes": 512 << 20}


def device_info():
    import torch

    p = torch.cuda.get_device_properties(0)
    info = {"arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "hip": torch.version.hip}
    name = p.name or torch.cuda.get_device_name(0)
    if name:  # empty where the marketing-name table is not installed
        info["name"] = name
    return info


def cpu_model():
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def settle(step, target_ms):
    """Back-to-back launches, in timed batches of 20, until about target_ms of
    GPU time has passed, so that the clock has reached its sustained level
    before the warm-up and the timed steps.  Reported in the output line;
    never part of the timed region."""
    import torch

    total, launches = 0.0, 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    while total < target_ms and launches < 100000:
        e0.record()
        for _ in range(20):
            step()
        e1.record()
        torch.cuda.synchronize()
        total += e0.elapsed_time(e1)
        launches += 20
    return {"ms": round(total, 2), "launches": launches}


def cpu_baseline(w, target_s):
    """Time the fp64 oracle on a bounded, seeded sample of the workload: whole
    (batch, head) slices in a seeded order until about target_s of wall time."""
    import numpy as np

    import oracle
    from synth_inputs import normal_qkv, to_bf16

    oracle.use_native_build()
    if w.backward:
        q, k, v, dout = normal_qkv(w.B, w.H, w.N, w.d, w.seed, with_dout=True)
    else:
        q, k, v = normal_qkv(w.B, w.H, w.N, w.d, w.seed, outliers=w.outliers)
    order = np.random.Generator(np.random.PCG64(12345)).permutation(w.B * w.H)
    flops_per_head = w.flops / (w.B * w.H)
    done, t_total = 0, 0.0
    for bh in order:
        b, h = divmod(int(bh), w.H)
        if w.dtype == "bf16":
            ref = [to_bf16(x[b:b + 1, h:h + 1])[1] for x in (q, k, v)]
        else:
            ref = [x[b:b + 1, h:h + 1] for x in (q, k, v)]
        t0 = time.perf_counter()
        if w.backward:
            d1 = dout[b:b + 1, h:h + 1]
            oracle.attn_bwd(*ref, to_bf16(d1)[1] if w.dtype == "bf16" else d1, causal=w.causal)
        else:
            oracle.attn_fwd(*ref, causal=w.causal)
        t_total += time.perf_counter() - t0
        done += 1
        if t_total >= target_s:
            break
    return {"value": done * flops_per_head / t_total / 1e12, "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "cpu": cpu_model(), "build": "gcc " + " ".join(oracle.NATIVE_CFLAGS),
            "kind": "oracle", "seconds": round(t_total, 3),
            "sample": f"{done} of {w.B * w.H} (batch, head) slices of the workload, every row, "
                      + ("fp64 analytic gradient, OpenMP over rows" if w.backward
                         else "fp64 two-pass, OpenMP over rows")}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(head sharding needs no communication; see the design notes). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_attention_77_amd as fa
    from synth_inputs import WORKLOADS, normal_qkv, to_bf16

    w = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if w.parts:
        return bench_merge(args, w, dev)
    if w.backward:
        q, k, v, dout = normal_qkv(w.B, w.H, w.N, w.d, w.seed, with_dout=True)
        dout = (to_bf16(dout)[0] if w.dtype == "bf16" else torch.from_numpy(dout)).to(dev)
    else:
        q, k, v = normal_qkv(w.B, w.H, w.N, w.d, w.seed, outliers=w.outliers)
    extra = {}
    if w.dtype == "fp8":
        from synth_inputs import hadamard_signs
        signs = torch.from_numpy(hadamard_signs(w.d)).to(dev)
        xs = [torch.from_numpy(x).to(dev) for x in (q, k, v)]

        def prepass():
            q8, qs = fa.flash_attn_fp8_quantize(xs[0], fa.ROLE_Q, rotate=True, signs=signs)
            k8, ks = fa.flash_attn_fp8_quantize(xs[1], fa.ROLE_K, rotate=True, signs=signs)
            v8, vs = fa.flash_attn_fp8_quantize(xs[2], fa.ROLE_V)
            return q8, k8, v8, qs, ks, vs
        for _ in range(3):
            prepass()
        torch.cuda.synchronize()
        # Ten rounds of the three calls.  Host-side marshalling takes about as
        # long as one call's kernel, so first the GPU is kept busy with a
        # bounded spin (torch.cuda._sleep) while the rounds are enqueued; they
        # then run back to back and the events time the kernels, not the host.
        def timed_rounds(n, ahead):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            if ahead:
                try:
                    torch.cuda._sleep(int(5e6))    # about 2.5 ms of spinning, bounded
                except (AttributeError, RuntimeError):
                    pass
            e0.record()
            for _ in range(n):
                out = prepass()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n, out
        pp_ms, f8 = timed_rounds(10, True)
        extra["prepass_host_bound_ms"] = round(timed_rounds(10, False)[0], 5)   # launched one by one
        # algorithmic bytes of the three pre-pass calls: fp32 Q, K, V read once,
        # e4m3 codes written (Q: the code and its residual term; V transposed
        # and padded to 64 keys), fp32 scales
        elems, npad = w.B * w.H * w.N * w.d, (w.N + 63) // 64 * 64
        pp_bytes = (3 * elems * 4 + 3 * elems + w.B * w.H * w.d * npad
                    + 4 * w.B * w.H * (2 * ((w.N + 31) // 32) + npad // 64))
        extra["prepass_ms"] = round(pp_ms, 5)
        extra["prepass_roofline"] = {"bound": "hbm", "achieved": round(pp_bytes / (pp_ms * 1e-3) / 1e9, 1),
                                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                     "frac": round(pp_bytes / (pp_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                     "bytes": pp_bytes}
        o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device=dev)
        del xs
    else:
        if w.dtype == "bf16":
            tens = [to_bf16(x)[0].to(dev) for x in (q, k, v)]
        else:
            tens = [torch.from_numpy(x).to(dev) for x in (q, k, v)]
        o = torch.empty_like(tens[0])
    del q, k, v
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    if w.backward:  # O and LSE of the forward feed every backward step
        fa.flash_attn_fwd(*tens, causal=w.causal, scale=w.scale, out=o, lse=lse)
        grads = [torch.empty_like(tens[0]) for _ in range(3)]
        lay = fa.Layout(w.B, w.H, w.N, w.d, *tens[0].stride()[:3])
        ws = torch.empty(fa.flash_attn_bwd_workspace_size(lay, fa.DTYPE_BF16 if w.dtype == "bf16" else fa.DTYPE_F32),
                         dtype=torch.uint8, device=dev)

    def step():
        if w.backward:
            fa.flash_attn_bwd(*tens, o, lse, dout, causal=w.causal, scale=w.scale,
                              dq=grads[0], dk=grads[1], dv=grads[2], workspace=ws)
        elif w.dtype == "fp8":
            fa.flash_attn_fwd_fp8(*f8, causal=w.causal, scale=w.scale, tile_cfg=args.tile_cfg,
                                  out=o, lse=lse)
        else:
            fa.flash_attn_fwd(*tens, causal=w.causal, scale=w.scale, tile_cfg=args.tile_cfg,
                              out=o, lse=lse)

    settled = settle(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"# settle {settled['ms']} ms ({settled['launches']} launches), warmup done "
          f"({args.warmup} steps), timing {args.steps} steps", file=sys.stderr, flush=True)

    # Timed region: K back-to-back launches on the current stream, bracketed by
    # synchronisation; HIP events on the same stream give the kernel's time.
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_ev = ev0.elapsed_time(ev1) / args.steps
    ms_wall = wall * 1e3 / args.steps
    ms = max(ms_ev, ms_wall)
    tflops = w.flops / (ms * 1e-3) / 1e12
    kernel_tflops = w.flops / (ms_ev * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    timing = launch_stats(step, stream, dev, min(50, args.steps))
    if w.dtype == "fp8":
        # the faster form that uses Q's first e4m3 term only (opts.fp8_q_terms = 1)
        def step1():
            fa.flash_attn_fwd_fp8(*f8, causal=w.causal, scale=w.scale, tile_cfg=args.tile_cfg,
                                  out=o, lse=lse, q_terms=1)
        for _ in range(max(args.warmup, 20)):
            step1()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            step1()
        e1.record(stream)
        torch.cuda.synchronize()
        ms1 = e0.elapsed_time(e1) / args.steps
        extra["one_term_q"] = {"ms_per_step": round(ms1, 5), "tflops": round(w.flops / (ms1 * 1e-3) / 1e12, 2)}

    out = {
        "metric": METRIC if w.name == "bf16_causal_n8192_d128" else
                  f"attention {'bwd' if w.backward else 'fwd'} TFLOP/s ({w.name})",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": ("synthetic (seeded N(0,1), 0.1% x20 outliers, fp32 -> e4m3 pre-pass)"
                 if w.dtype == "fp8" else "synthetic (seeded N(0,1), bf16-rounded)" if w.dtype == "bf16"
                 else "synthetic (seeded N(0,1), fp32)"),
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "seq_len": w.N,
                   "head_dim": w.d, "causal": w.causal, "scale": w.scale,
                   "flop_per_step": w.flops, "tile_cfg": args.tile_cfg},
        "pct_of_peak": round(100.0 * tflops / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(kernel_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(kernel_tflops / peak, 4),
                     "traffic": measured_traffic(w), "kernel_ms": round(ms_ev, 5)},
        "timing": timing,
        "settle": settled,
        "device": device_info(),
    }
    out.update(extra)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = n * 4
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def bench_merge(args, w, dev):
    """The (O, LSE) merge: an HBM stream, reported in GB/s of algorithmic bytes."""
    import numpy as np
    import torch

    import exact_attention_77_amd as fa
    from synth_inputs import merge_parts

    o_parts, lse_parts = merge_parts(w, dev)
    o = torch.empty(o_parts.shape[1:], dtype=o_parts.dtype, device=dev)
    lse = torch.empty(lse_parts.shape[1:], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        fa.flash_attn_merge(o_parts, lse_parts, out=o, lse=lse)

    settled = settle(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_ev = ev0.elapsed_time(ev1) / args.steps
    ms = max(ms_ev, (time.perf_counter() - t0) * 1e3 / args.steps)
    gbs = w.merge_bytes / (ms * 1e-3) / 1e9
    kgbs = w.merge_bytes / (ms_ev * 1e-3) / 1e9
    timing = launch_stats(step, stream, dev, min(50, args.steps))
    out = {
        "metric": f"attention merge GB/s ({w.name})", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded device draws: O ~ N(0,1) bf16, LSE ~ 7 + 2 N(0,1))",
        "config": {"workload": w.name, "parts": w.parts, "batch": w.B, "heads": w.H, "seq_len": w.N,
                   "head_dim": w.d, "bytes_per_step": w.merge_bytes},
        "roofline": {"bound": "hbm", "achieved": round(kgbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(kgbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic(w),
                     "kernel_ms": round(ms_ev, 5)},
        "timing": timing,
        "settle": settled,
        "device": device_info(),
    }
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = n * 4
    if not args.no_cpu_baseline:
        import oracle
        S, B, H, N, d = o_parts.shape
        order = np.random.Generator(np.random.PCG64(12345)).permutation(B * H)
        done, t_total = 0, 0.0
        for bh in order:
            b, h = divmod(int(bh), H)
            op = o_parts[:, b, h].float().cpu().numpy()
            lp = lse_parts[:, b, h].cpu().numpy()
            t1 = time.perf_counter()
            oracle.merge(op, lp)
            t_total += time.perf_counter() - t1
            done += 1
            if t_total >= args.cpu_seconds:
                break
        out["cpu_baseline"] = {"value": round(done * w.merge_bytes / (B * H) / t_total / 1e9, 3),
                               "unit": "GB/s", "cores": 1, "kind": "oracle",
                               "seconds": round(t_total, 3),
                               "sample": f"{done} of {B * H} (batch, head) slices, every row, fp64 numpy"}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
