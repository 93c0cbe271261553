"""Benchmark: Muon optimizer steps/s on the MoE expert batch 256 x (2048 x 7168) bf16.

One step = the whole hot path over all 256 matrices: momentum + Nesterov
input + ||N||_F, normalisation, 10 hybrid Newton-Schulz iterations (each a
grouped X X^T, A A and (aI + bA + cA^2) X launch) and the fused rescale,
decay and update.  Inputs are synthetic (seeded, generated on the device with
the low-rank-plus-noise gradient law) and resident in HBM before timing.

Prints one JSON line.  `roofline` reports the dominant kernel (most total
time) with its algorithmic FLOPs (or bytes) per launch divided by its average
launch duration, measured with HIP events on the stream it runs on.
`cpu_baseline` times the CPU oracle on one of the 256 matrices and scales to
a step.
"""

import argparse
import hashlib
import json
import math
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Muon optimizer steps/sec + NS TFLOP/s (% bf16 MFMA peak), 256×(2048×7168) batch"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
NS_STAGES = ("gram", "poly", "apply", "apply_update")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_moe_256x2048x7168.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_source_sha():
    """Hash of the bf16 Newton-Schulz kernel sources (comments and blank
    space removed) the stored traffic counters were taken on."""
    h = hashlib.sha256()
    for name in ("ns_gemm_bf16.hip", "common.hpp"):
        with open(os.path.join(ROOT, "muon_step_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def copy_calibration():
    """A plain 1 GiB device-to-device copy: the reference for scaling FETCH_SIZE
    and WRITE_SIZE (profile this mode with rocprofv3 --pmc)."""
    import torch
    x = torch.full((1 << 28,), 1.0, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": x.numel() * 4}), flush=True)


def library_baseline(rows, cols, count):
    """torch (hipBLASLt) bf16 batched products of the three Newton-Schulz
    shapes over `count` matrices, dense and with contiguous operands: a
    reference point for the fused kernels, not part of the Muon step."""
    import torch
    s, l = min(rows, cols), max(rows, cols)
    g = torch.Generator(device="cuda").manual_seed(0)
    x = (torch.randn(count, s, l, device="cuda", generator=g) * 0.01).to(torch.bfloat16)
    xt = x.transpose(1, 2).contiguous()
    b = (torch.randn(count, s, s, device="cuda", generator=g) * 0.01).to(torch.bfloat16)
    out = {}
    for name, fn, flops in (("apply B@X", lambda: torch.bmm(b, x), 2.0 * count * s * s * l),
                            ("gram X@X^T", lambda: torch.bmm(x, xt), 2.0 * count * s * s * l),
                            ("poly B@B", lambda: torch.bmm(b, b), 2.0 * count * s * s * s)):
        fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(5):
            fn()
        t1.record()
        t1.synchronize()
        ms = t0.elapsed_time(t1) / 5
        out[name] = {"ms": round(ms, 4), "dense_tflops": round(flops / ms / 1e9, 1)}
    print(json.dumps({"library_bmm_bf16": out, "matrices": count, "shape": [s, l]}), flush=True)


def adamw_rate(ctx, torch, ms, stream, steps=5):
    """The AdamW path on the 16B-MoE workload's embedding and head (two
    102400 x 2048 fp32 tensors, 28 bytes per element per step), timed with the
    library's per-launch events."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    tens = []
    for _ in range(2):
        shape = (102400, 2048)
        p = torch.randn(shape, generator=gen, device="cuda") * 0.02
        g = torch.randn(shape, generator=gen, device="cuda") * 1e-3
        tens.append((p, g, torch.zeros_like(p), torch.zeros_like(p)))
    descs = [ms.adamw_tensor(*t) for t in tens]
    ctx.muon_adamw_step(descs, ms.adamw_hparams(step=1), stream)
    torch.cuda.synchronize()
    ctx.muon_profile_enable(True)
    for i in range(steps):
        ctx.muon_adamw_step(descs, ms.adamw_hparams(step=i + 2), stream)
    torch.cuda.synchronize()
    st = ctx.muon_profile_read()["adamw"]
    ctx.muon_profile_enable(False)
    gbs = st["bytes"] / st["total_ms"] / 1e6
    log(f"  adamw              launches {st['launches']:5d}  avg {st['total_ms'] / st['launches']:9.4f} ms  "
        f"{gbs:8.1f} GB/s")
    del tens, descs
    return {"GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "ms_per_step": round(st["total_ms"] / st["launches"], 4),
            "workload": "embedding + head, 2 x 102400x2048 fp32, 28 B/elem"}


PROBE_MIX = {"momentum_nesterov": (6, 7), "adamw": (4, 3), "update": (5, 2), "copy": (1, 1)}


def hbm_probe(ctx, torch, stream, stream_bytes=1 << 30, steps=5):
    """The library's streaming probe at each elementwise kernel's read : write mix
    (streams of 1 GiB, every 16-byte vector read or written once, 1 GiB + 197,632
    bytes apart so that the streams do not start at power-of-two distances, as
    separate allocations do not), timed with its per-launch events: the HBM
    ceiling those kernels are compared with."""
    out = {}
    pitch = stream_bytes + 12352 * 16
    for name, (r, w) in PROBE_MIX.items():
        src = torch.empty((r - 1) * pitch + stream_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty((w - 1) * pitch + stream_bytes, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        ctx.muon_stream_probe(src, dst, stream_bytes, r, w, pitch, stream)
        torch.cuda.synchronize()
        ctx.muon_profile_enable(True)
        for _ in range(steps):
            ctx.muon_stream_probe(src, dst, stream_bytes, r, w, pitch, stream)
        torch.cuda.synchronize()
        st = ctx.muon_profile_read()["stream_probe"]
        ctx.muon_profile_enable(False)
        gbs = st["bytes"] / st["total_ms"] / 1e6
        log(f"  probe {r}:{w} ({name:17s}) avg {st['total_ms'] / st['launches']:8.4f} ms  {gbs:8.1f} GB/s")
        out[name] = {"reads_writes": [r, w], "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
        del src, dst
        torch.cuda.empty_cache()
    return out


def moe16b_step(args):
    """Times the full synthetic 16B-MoE optimizer step (27 layers: 4 x 2048^2
    attention matrices and 64 experts x (2048x1408 up, gate; 1408x2048 down),
    Muon on all 5292 matrices in one call, then AdamW on the 102400x2048
    embedding and head) and prints one JSON line of its own."""
    import torch

    import muon_step_amd as ms
    import synth

    wl = synth.WORKLOADS["moe16b_full_step"]
    specs = list(wl.matrices)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.base_seed)
    log(f"generating the 16B-MoE step: {len(specs)} Muon matrices + AdamW")
    by_shape = {}
    for i, sp in enumerate(specs):
        by_shape.setdefault((sp.rows, sp.cols), []).append(i)
    grads = [None] * len(specs)
    for (rows, cols), ids in by_shape.items():
        g = synth.spectral_grad_torch(rows, cols, len(ids), gen, "cuda")
        for k, i in enumerate(ids):
            grads[i] = g[k]
    params = [(torch.randn(sp.rows, sp.cols, generator=gen, device="cuda") * synth.gen.PARAM_STD).to(torch.bfloat16)
              for sp in specs]
    moms = [torch.zeros(sp.rows, sp.cols, device="cuda") for sp in specs]
    mats = [ms.matrix(params[i], grads[i], moms[i]) for i in range(len(specs))]
    adamw_bufs = []  # the descriptors hold raw pointers: keep every tensor alive
    for _, n in wl.adamw:
        p = torch.randn(n, generator=gen, device="cuda") * synth.gen.PARAM_STD
        adamw_bufs.append((p, torch.randn(n, generator=gen, device="cuda") * 1e-3, torch.zeros_like(p),
                           torch.zeros_like(p)))
    tensors = [ms.adamw_tensor(*b) for b in adamw_bufs]
    hp = ms.make_hparams(lr=0.02, momentum=0.95, weight_decay=0.1, gamma=0.2, nesterov=True,
                         ns_precision=ms.MUON_NS_BF16,
                         scale_mode=ms.MUON_SCALE_UNIT_RMS if args.scale_mode == "unit_rms" else ms.MUON_SCALE_SQRT_MAX)
    ctx = ms.Context(0, args.workspace_gib << 30)
    stream = torch.cuda.current_stream()

    def step(i):
        ctx.muon_step(mats, hp, stream)
        ctx.muon_adamw_step(tensors, ms.adamw_hparams(step=i + 1), stream)

    for i in range(args.warmup):
        step(i)
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")
    ctx.muon_profile_enable(True)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    stop.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(stop) / args.steps
    stages = ctx.muon_profile_read()
    ctx.close()
    ns_ms = sum(stages[k]["total_ms"] for k in NS_STAGES if k in stages)
    ns_flops = sum(stages[k]["flops"] for k in NS_STAGES if k in stages)
    breakdown = {k: round(v["total_ms"] / args.steps, 3) for k, v in stages.items()}
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step; per stage (ms/step): {breakdown}")
    print(json.dumps({
        "metric": "16B-MoE optimizer step (Muon on 5292 matrices + AdamW on embedding and head)",
        "value": round(1000.0 / ms_per_step, 4), "unit": "steps/s", "ms_per_step": round(ms_per_step, 3),
        "steps": args.steps, "warmup": args.warmup, "n_gpus": 1, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "moe16b_full_step", "muon_matrices": len(specs),
                   "workspace_cap_gib": args.workspace_gib, "scale_mode": args.scale_mode},
        "ns_tflops": round(ns_flops / ns_ms / 1e9, 2) if ns_ms else None,
        "ns_frac_bf16_peak": round(ns_flops / ns_ms / 1e9 / PEAK_BF16_TFLOPS, 4) if ns_ms else None,
        "stage_ms_per_step": breakdown}), flush=True)


def workload_step(args):
    """Times one Muon step over a listed workload (the dense block: 4 x 4096^2,
    2 x 4096x14336, 14336x4096; or the aspect-ratio set: 1024x16384, 16384x1024,
    7168^2, 512x32768 with pre-filled momentum), all matrices in one call, and
    prints one JSON line of its own: ms/step, NS TFLOP/s on the algorithmic
    count and its fraction of the bf16 peak, per-stage times and the
    elementwise kernels' GB/s."""
    import torch

    import muon_step_amd as ms
    import synth

    wl = synth.WORKLOADS[args.workload]
    specs = list(wl.matrices)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.base_seed)
    log(f"generating {wl.name}: {len(specs)} matrices")
    by_shape = {}
    for i, sp in enumerate(specs):
        by_shape.setdefault((sp.rows, sp.cols), []).append(i)
    grads, moms = [None] * len(specs), [None] * len(specs)
    for (rows, cols), ids in by_shape.items():
        g = synth.spectral_grad_torch(rows, cols, len(ids), gen, "cuda")
        pf = [i for i in ids if specs[i].prefill_momentum]
        gp = synth.spectral_grad_torch(rows, cols, len(pf), gen, "cuda") if pf else None
        for k, i in enumerate(ids):
            grads[i] = g[k]
        for k, i in enumerate(pf):
            moms[i] = gp[k].float()
    params = [(torch.randn(sp.rows, sp.cols, generator=gen, device="cuda") * synth.gen.PARAM_STD).to(torch.bfloat16)
              for sp in specs]
    moms = [m if m is not None else torch.zeros(sp.rows, sp.cols, device="cuda") for sp, m in zip(specs, moms)]
    mats = [ms.matrix(params[i], grads[i], moms[i]) for i in range(len(specs))]
    hp = ms.make_hparams(lr=0.02, momentum=0.95, weight_decay=0.1, gamma=0.2, nesterov=True,
                         ns_precision=ms.MUON_NS_BF16,
                         scale_mode=ms.MUON_SCALE_UNIT_RMS if args.scale_mode == "unit_rms" else ms.MUON_SCALE_SQRT_MAX)
    ctx = ms.Context(0)
    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        ctx.muon_step(mats, hp, stream)
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed_steps():
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(args.steps):
            ctx.muon_step(mats, hp, stream)
        stop.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / args.steps

    # the step as a caller runs it (groups of different shapes concurrently),
    # then with the groups in turn, and once more under per-stage timing (which
    # runs them in turn) for the breakdown
    ms_per_step = timed_steps()
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step")
    ctx.muon_set_concurrent_groups(False)
    ms_in_turn = timed_steps()
    log(f"timed {args.steps} steps with the groups in turn: {ms_in_turn:.3f} ms/step")
    ctx.muon_profile_enable(True)
    timed_steps()
    stages = ctx.muon_profile_read()
    ctx.close()
    for name, st in stages.items():
        rate = (f"{st['flops'] / st['total_ms'] / 1e9:8.1f} TFLOP/s" if st["flops"] else
                f"{st['bytes'] / st['total_ms'] / 1e6:8.1f} GB/s" if st["total_ms"] else "")
        log(f"  {name:18s} launches {st['launches']:5d}  total/step {st['total_ms'] / args.steps:9.3f} ms  {rate}")
    ns_ms = sum(stages[k]["total_ms"] for k in NS_STAGES if k in stages)
    ns_flops = sum(stages[k]["flops"] for k in NS_STAGES if k in stages)
    ns_tflops = ns_flops / ns_ms / 1e9 if ns_ms else 0.0
    dense = sum(10 * 2 * (2 * max(sp.rows, sp.cols) * min(sp.rows, sp.cols) ** 2 + min(sp.rows, sp.cols) ** 3)
                for sp in specs)
    elementwise = {}
    for k in ("momentum_nesterov", "normalize", "unit_rms", "update"):
        if k in stages and stages[k]["total_ms"] and stages[k]["bytes"]:
            gbs = stages[k]["bytes"] / stages[k]["total_ms"] / 1e6
            elementwise[k] = {"GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                              "ms_per_step": round(stages[k]["total_ms"] / args.steps, 4)}
    print(json.dumps({
        "metric": f"Muon optimizer steps/sec + NS TFLOP/s (% bf16 MFMA peak), {wl.name}",
        "value": round(1000.0 / ms_per_step, 4), "unit": "steps/s", "ms_per_step": round(ms_per_step, 3),
        "ms_per_step_groups_in_turn": round(ms_in_turn, 3),
        "steps": args.steps, "warmup": args.warmup, "n_gpus": 1, "dtype": "bf16",
        "data": "synthetic (seeded low-rank-plus-noise bf16 gradients, N(0,0.02) bf16 params)",
        "config": {"workload": wl.name, "matrices": [[sp.rows, sp.cols] for sp in specs], "ns_steps": 10,
                   "scale_mode": args.scale_mode},
        "ns_tflops": round(ns_tflops, 2), "ns_frac_bf16_peak": round(ns_tflops / PEAK_BF16_TFLOPS, 4),
        "ns_dense_equivalent_tflops": round(dense * args.steps / ns_ms / 1e9, 2) if ns_ms else None,
        "ns_ms_per_step": round(ns_ms / args.steps, 3),
        "elementwise": elementwise,
        "stage_ms_per_step": {k: round(v["total_ms"] / args.steps, 4) for k, v in stages.items()}}), flush=True)


def cpu_baseline(rows, cols, count, scale_mode="sqrt_max"):
    """The oracle as it stands on one matrix of the batch; scaled to one step."""
    import numpy as np

    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    wl = synth.Workload("moe_256x2048x7168_bf16", 4, (synth.MatrixSpec(rows, cols),))
    inp = synth.matrix_inputs(wl, 0)
    t0 = time.perf_counter()
    oracle.muon_step(inp["w"], inp["g"], inp["m"], param_bf16=True, scale_mode=scale_mode)
    dt = time.perf_counter() - t0
    return {"value": 1.0 / (dt * count), "unit": "steps/s", "cores": int(cores), "kind": "oracle",
            "sample": f"1 of {count} matrices ({rows}x{cols}), full oracle step (fp32 bookkeeping, fp64 "
                      f"Newton-Schulz) in {dt:.2f} s, scaled x{count}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--experts", type=int, default=256)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB copy (reference for the HBM byte counters)")
    ap.add_argument("--workload", default="moe_256x2048x7168_bf16",
                    choices=["moe_256x2048x7168_bf16", "moe16b", "dense_block_bf16", "aspect_stress_bf16"],
                    help="moe16b: time the full 16B-MoE optimizer step instead; dense_block_bf16, "
                         "aspect_stress_bf16: one step over that matrix set (each its own JSON line)")
    ap.add_argument("--workspace-gib", type=int, default=64, help="NS workspace cap for --workload moe16b")
    ap.add_argument("--scale-mode", default="sqrt_max", choices=["sqrt_max", "unit_rms"],
                    help="update scale: sqrt(max(n,m))*gamma (DeepSeek-V4) or the unit-RMS mode")
    ap.add_argument("--library-baseline", action="store_true",
                    help="only time torch bf16 batched products of the same shapes (64 matrices)")
    ap.add_argument("--hbm-probe", action="store_true",
                    help="only time the library's streaming probe at the elementwise kernels' read:write mixes")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.library_baseline:
        library_baseline(2048, 7168, 64)
        return
    if args.hbm_probe:
        import torch

        import muon_step_amd as ms
        ctx = ms.Context(0)
        print(json.dumps({"hbm_probe": hbm_probe(ctx, torch, torch.cuda.current_stream())}), flush=True)
        ctx.close()
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the per-GPU work of a sharded "
              "run is the same grouped kernel on that GPU's share of matrices); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.workload == "moe16b":
        moe16b_step(args)
        return
    if args.workload in ("dense_block_bf16", "aspect_stress_bf16"):
        workload_step(args)
        return

    import torch

    import muon_step_amd as ms
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    rows, cols, count = 2048, 7168, args.experts
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    log(f"generating {count} x {rows}x{cols} bf16 inputs on the device")
    grads = synth.spectral_grad_torch(rows, cols, count, gen, "cuda")
    params = (torch.randn(count, rows, cols, generator=gen, device="cuda") * synth.gen.PARAM_STD).to(torch.bfloat16)
    moms = torch.zeros(count, rows, cols, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    mats = [ms.matrix(params[e], grads[e], moms[e]) for e in range(count)]
    hp = ms.make_hparams(lr=0.02, momentum=0.95, weight_decay=0.1, gamma=0.2, nesterov=True,
                         ns_precision=ms.MUON_NS_BF16,
                         scale_mode=ms.MUON_SCALE_UNIT_RMS if args.scale_mode == "unit_rms" else ms.MUON_SCALE_SQRT_MAX)
    ctx = ms.Context(0)
    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        ctx.muon_step(mats, hp, stream)
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")
    ctx.muon_profile_enable(True)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        ctx.muon_step(mats, hp, stream)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    stages = ctx.muon_profile_read()
    ctx.muon_profile_enable(False)
    ms_per_step = total_ms / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step")
    for name, st in stages.items():
        avg = st["total_ms"] / st["launches"]
        rate = (f"{st['flops'] / st['total_ms'] / 1e9:8.1f} TFLOP/s" if st["flops"] else
                f"{st['bytes'] / st['total_ms'] / 1e6:8.1f} GB/s")
        log(f"  {name:18s} launches {st['launches']:5d}  avg {avg:9.4f} ms  total/step "
            f"{st['total_ms'] / args.steps:9.3f} ms  {rate}")

    ns_ms = sum(stages[k]["total_ms"] for k in NS_STAGES if k in stages)
    ns_flops = sum(stages[k]["flops"] for k in NS_STAGES if k in stages)
    ns_tflops = ns_flops / ns_ms / 1e9 if ns_ms else 0.0
    dense_flops_step = count * 10 * 2 * (2 * cols * rows * rows + rows ** 3)
    dom_name = max(stages, key=lambda k: stages[k]["total_ms"])
    dom = stages[dom_name]
    avg_ms = dom["total_ms"] / dom["launches"]
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_stage") == dom_name and tr.get("source_sha256") == gemm_source_sha():
            traffic = tr.get("hbm_bytes_per_launch")
    # the bytes the dominant kernel must move at least once per launch (its
    # operands once, X_lo, and X_hi + X_lo out for the apply product)
    compulsory = dom["bytes"] / dom["launches"]
    if dom["flops"]:
        achieved = dom["flops"] / dom["launches"] / (avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": dom_name, "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "traffic_compulsory": compulsory, "flops_per_launch": dom["flops"] / dom["launches"],
                "avg_launch_ms": round(avg_ms, 4)}
    else:
        achieved = dom["bytes"] / dom["launches"] / (avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": dom_name, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "traffic_compulsory": compulsory, "bytes_per_launch": dom["bytes"] / dom["launches"],
                "avg_launch_ms": round(avg_ms, 4)}
    elementwise = {}
    for k in ("momentum_nesterov", "normalize", "unit_rms", "update"):
        if k in stages and stages[k]["total_ms"] and stages[k]["bytes"]:
            gbs = stages[k]["bytes"] / stages[k]["total_ms"] / 1e6
            elementwise[k] = {"GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                              "ms_per_step": round(stages[k]["total_ms"] / args.steps, 4)}
    out = {
        "metric": METRIC,
        "value": round(1000.0 / ms_per_step, 4),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded low-rank-plus-noise bf16 gradients, N(0,0.02) bf16 params, zero fp32 momentum)",
        "config": {"workload": "moe_256x2048x7168_bf16", "matrices": count, "shape": [rows, cols],
                   "ns_steps": 10, "schedule": "deepseekv4 8x(3.4445,-4.7750,2.0315)+2x(2,-1.5,0.5)",
                   "ns_precision": "bf16 MFMA operands, fp32 accumulate, X kept as bf16 hi + 8-bit residual",
                   "lr": 0.02, "momentum": 0.95, "weight_decay": 0.1, "gamma": 0.2,
                   "scale_mode": args.scale_mode},
        "ns_tflops": round(ns_tflops, 2),
        "ns_frac_bf16_peak": round(ns_tflops / PEAK_BF16_TFLOPS, 4),
        "ns_dense_equivalent_tflops": round(dense_flops_step * args.steps / ns_ms / 1e9, 2) if ns_ms else None,
        "ns_ms_per_step": round(ns_ms / args.steps, 3),
        "elementwise": elementwise,
        "roofline": roof,
        "cpu_baseline": None,
        "pages_context": "NS adds ~5% training FLOPs (DeepSeek-V4 book ch. 6; no hardware given)",
    }
    del grads, params, moms, mats
    torch.cuda.empty_cache()
    out["elementwise"]["adamw"] = adamw_rate(ctx, torch, ms, stream)
    probe = hbm_probe(ctx, torch, stream)
    for k, v in out["elementwise"].items():
        if k in probe:
            v["frac_of_probe"] = round(v["GB/s"] / probe[k]["GB/s"], 4)
    out["hbm_probe"] = probe
    ctx.close()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on one matrix")
        out["cpu_baseline"] = cpu_baseline(rows, cols, count, args.scale_mode)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
