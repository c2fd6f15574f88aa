"""Benchmark of the ternary-weight matmul on one MI355X.

Default workload: 27B-class attention-projection decode, M=1, K=N=5120,
bf16 activations, 2-bit packed weights with one fp16 scale per 128 weights,
bf16 output.  One step = one tern_matmul call (the whole per-token hot path
of that projection: stream the packed weights and scales, decode, sign-select
accumulate, scale at block boundaries, reduce, round, store).  Weight copies
rotate through >= 2 GB of distinct device buffers so that no step finds its
weights in the 256 MB last-level cache; inputs are resident in HBM before
timing starts.

Prints ONE JSON line (rank 0).  `value` is packed-weight GB/s for M=1 decode
configurations and TFLOP/s for batched ones, as the metric defines them.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, vendor figure
METRIC = ("packed-weight GB/s & % HBM peak (M=1 GEMV); TFLOP/s & % MFMA peak (M≥256)")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--config", type=int, default=2, help="workload id (workloads.CONFIGS)")
    ap.add_argument("--shape", type=int, default=0, help="shape index inside the workload")
    ap.add_argument("--path", default="auto", choices=["auto", "gemv", "mfma", "gemv_mfma", "gemv_fp4"])
    ap.add_argument("--rotate-gb", type=float, default=2.0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate", action="store_true",
                    help="measure the per-launch floor (a one-element kernel) and plain copy bandwidth")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the comparison route, the other workloads and the decode sweep")
    ap.add_argument("--eager", action="store_true",
                    help="launch each step from Python instead of replaying a captured HIP graph")
    return ap.parse_args()


def measured_traffic(workload_key: str):
    """HBM bytes per launch from the committed counter summary, if it still applies.

    profiles/traffic.json records FETCH_SIZE / WRITE_SIZE per dispatch (scaled
    by a copy kernel of known size) together with the sha256 of the kernel
    sources it was measured on.  If the sources changed since, the figure no
    longer describes this build and None is returned.
    """
    import hashlib

    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", "traffic.json")
    try:
        entry = json.load(open(path))[workload_key]
    except (OSError, KeyError, ValueError):
        return None
    m = hashlib.sha256()
    for src in entry["sources"]:
        try:
            m.update(open(os.path.join(root, src), "rb").read())
        except OSError:
            return None
    if m.hexdigest() != entry["sources_sha256"]:
        return None
    return int(entry["hbm_bytes_per_launch"])


def cpu_baseline(p, seconds: float):
    """The CPU oracle, as it stands, on a bounded sample of the same workload."""
    import oracle

    o = oracle.default()
    sh = p.shape
    cores = len(os.sched_getaffinity(0))
    threads = max(1, min(16, cores))
    # bounded sample: whole output columns of the problem, all rows m
    n_cols = sh.N if sh.M * sh.K * sh.N <= 3e8 else max(threads, int(3e8 // (sh.M * sh.K)))
    n_cols = min(n_cols, sh.N)
    sub = p.packed[:n_cols]
    ssc = p.scales[:n_cols]
    reps, t0 = 0, time.perf_counter()
    while True:
        o.matmul(p.x, p.x_dtype, sub, ssc, sh.M, n_cols, sh.K, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per = el / reps
    if sh.M == 1:
        val, unit = n_cols * sh.K / 4 / per / 1e9, "GB/s"
    else:
        val, unit = 2.0 * sh.M * n_cols * sh.K / per / 1e12, "TFLOP/s"
    sample = (f"{reps} full oracle passes over {n_cols} of {sh.N} output columns "
              f"(M={sh.M}, K={sh.K}), {el:.1f} s")
    return {"value": round(val, 6), "unit": unit, "cores": threads, "kind": "oracle", "sample": sample}


def calibrate(steps: int):
    """Per-launch floor and achievable bandwidth of plain torch kernels, same timing protocol."""
    import torch

    dev = torch.device("cuda:0")
    out = {"calibration": True}
    one = torch.zeros(1, device=dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            one.add_(1.0)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    out["one_element_kernel_us_per_launch_graph"] = round(a.elapsed_time(b) * 1e3 / steps, 4)
    for gb in (0.0066, 0.0223, 1.0):
        n = int(gb * 1e9) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        reps = 20 if gb >= 1 else 200
        copies = [torch.ones(n, dtype=torch.float32, device=dev) for _ in range(max(1, int(2.0 / gb)) if gb < 1 else 1)]
        dst.copy_(src)
        torch.cuda.synchronize()
        a.record()
        for i in range(reps):
            dst.copy_(copies[i % len(copies)])
        b.record()
        torch.cuda.synchronize()
        sec = a.elapsed_time(b) / 1e3 / reps
        out[f"copy_{gb:g}GB_read_plus_write_GBps"] = round(2 * n * 4 / sec / 1e9, 1)
        out[f"copy_{gb:g}GB_us"] = round(sec * 1e6, 3)
        del copies
    return out


def _tdt(name):
    import torch
    return {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[name]


def _device_problem(p, rotate_gb):
    """Device copies of a problem: X, Y and enough weight copies to span rotate_gb."""
    import numpy as np
    import torch

    dev = torch.device("cuda:0")
    sh = p.shape
    x = torch.from_numpy(p.x.view(np.int16)).to(dev).view(_tdt(p.x_dtype))
    w0 = torch.from_numpy(p.packed).to(dev)
    s0 = torch.from_numpy(p.scales.view(np.int16)).to(dev).view(torch.float16)
    wbytes = w0.numel() + s0.numel() * 2
    copies = max(1, int(np.ceil(rotate_gb * 1e9 / wbytes)))
    ws = [w0] + [w0.clone() for _ in range(copies - 1)]
    ss = [s0] + [s0.clone() for _ in range(copies - 1)]
    y = torch.empty((sh.M, sh.N), dtype=_tdt(p.y_dtype), device=dev)
    return x, ws, ss, y, copies, wbytes


def _graph_time_ms(step, steps, warmup):
    """ms per step of `steps` calls captured in one HIP graph (after warm-up)."""
    import torch

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            step(warmup + i)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def _summary(p, ms):
    sh = p.shape
    sec = ms / 1e3
    yb = {"f32": 4, "bf16": 2, "f16": 2}[p.y_dtype]
    alg = sh.N * sh.K / 4 + sh.N * sh.K / 64 + 2 * sh.M * sh.K + yb * sh.M * sh.N
    out = {"M": sh.M, "K": sh.K, "N": sh.N, "us_per_launch": round(ms * 1e3, 3),
           "packed_GBps": round(sh.N * sh.K / 4 / sec / 1e9, 1),
           "alg_GBps": round(alg / sec / 1e9, 1), "TFLOPs": round(2.0 * sh.M * sh.N * sh.K / sec / 1e12, 2)}
    if sh.M <= 16:
        out["roofline"] = {"bound": "hbm", "frac": round(alg / sec / 1e9 / HBM_PEAK_GBS, 4)}
    else:
        out["roofline"] = {"bound": "mfma", "frac": round(2.0 * sh.M * sh.N * sh.K / sec / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}
    return out


def other_workloads(skip):
    """Every configured shape except the headline one, same protocol, fewer steps."""
    import torch

    import ternary_weight_matmul_amd as tern
    import workloads

    res = []
    for cid in (1, 2, 3, 4, 5):
        for si, sh in enumerate(workloads.CONFIGS[cid].shapes):
            if (cid, si) == skip:
                continue
            p = workloads.make_problem(cid, si)
            x, ws, ss, y, copies, _ = _device_problem(p, 1.0)
            big = sh.M * sh.N * sh.K > 1e10
            steps = 40 if big else (200 if sh.M > 16 else 500)
            ms = _graph_time_ms(lambda i: tern.matmul_into(x, ws[i % copies], ss[i % copies], y),
                                steps, 10)
            rec = {"workload": f"{workloads.CONFIGS[cid].name} ({sh.label})", **_summary(p, ms)}
            res.append(rec)
            del x, ws, ss, y
            torch.cuda.empty_cache()
    return res


def comparison_route(cid, si):
    """The pages' first route: dequantise to 16-bit W, then a library GEMM (hipBLASLt via
    torch), against the fused kernel, on one workload (no weight rotation for either)."""
    import numpy as np
    import torch

    import ternary_weight_matmul_amd as tern
    import workloads

    p = workloads.make_problem(cid, si)
    sh = p.shape
    dev = torch.device("cuda:0")
    x = torch.from_numpy(p.x.view(np.int16)).to(dev).view(_tdt(p.x_dtype))
    w = torch.from_numpy(p.packed).to(dev)
    s = torch.from_numpy(p.scales.view(np.int16)).to(dev).view(torch.float16)
    wdt = _tdt(p.x_dtype)
    W = torch.empty((sh.N, sh.K), dtype=wdt, device=dev)
    xT = x.t().contiguous()                     # [K, M]: both GEMM operands contiguous
    yT = torch.empty((sh.N, sh.M), dtype=wdt, device=dev)
    y = torch.empty((sh.M, sh.N), dtype=_tdt(p.y_dtype), device=dev)
    steps = 20 if sh.M > 16 else 200
    t_deq = _graph_time_ms(lambda i: tern.dequant(w, s, out=W), steps, 5)
    t_gemm = _graph_time_ms(lambda i: torch.matmul(W, xT, out=yT), steps, 5)
    t_fused = _graph_time_ms(lambda i: tern.matmul_into(x, w, s, y), steps, 5)
    return {"workload": f"{workloads.CONFIGS[cid].name} M={sh.M} K={sh.K} N={sh.N}",
            "dequant_us": round(t_deq * 1e3, 3), "library_gemm_us": round(t_gemm * 1e3, 3),
            "route_total_us": round((t_deq + t_gemm) * 1e3, 3), "fused_us": round(t_fused * 1e3, 3),
            "route_over_fused": round((t_deq + t_gemm) / t_fused, 3),
            "dense_weight_bytes": int(sh.N * sh.K * 2), "packed_weight_bytes": int(sh.N * sh.K // 4),
            "note": "weights resident (no rotation) for both routes"}


def int8_scale_variant():
    """fp16 block scales vs int8 codes with a per-row fp32 factor (tern_matmul_s8) on the
    decode and batched shapes, same protocol (weights rotated over 1 GB)."""
    import torch

    import ternary_weight_matmul_amd as tern
    import workloads

    res = []
    for cid, si in ((2, 0), (3, 0), (3, 1), (3, 4), (4, 0)):
        p = workloads.make_problem(cid, si)
        sh = p.shape
        x, ws, ss, y, copies, _ = _device_problem(p, 1.0)
        qr = [tern.quantize_scales(s) for s in ss]
        steps = 100 if sh.M > 16 else 500
        t16 = _graph_time_ms(lambda i: tern.matmul_into(x, ws[i % copies], ss[i % copies], y), steps, 10)
        t8 = _graph_time_ms(lambda i: tern.matmul_s8_into(x, ws[i % copies], qr[i % copies][0],
                                                          qr[i % copies][1], y), steps, 10)
        packed = sh.N * sh.K // 4
        res.append({"workload": f"{workloads.CONFIGS[cid].name} M={sh.M} K={sh.K} N={sh.N}",
                    "fp16_scales_us": round(t16 * 1e3, 3), "int8_scales_us": round(t8 * 1e3, 3),
                    "int8_over_fp16": round(t8 / t16, 4),
                    "weight_bytes_fp16_scales": int(packed + sh.N * (sh.K // 128) * 2),
                    "weight_bytes_int8_scales": int(packed + sh.N * (sh.K // 128) + 4 * sh.N)})
        del x, ws, ss, y, qr
        torch.cuda.empty_cache()
    return res


def zero_block_skip(rate: float = 0.5):
    """Dense tern_matmul vs tern_matmul_blockmap on decode shapes whose weights have a
    fraction `rate` of all-zero 128-weight blocks (and on the dense weights, rate 0,
    for the skipping kernel's overhead); weights rotated over 1 GB."""
    import numpy as np
    import torch

    import ternary_weight_matmul_amd as tern
    import workloads

    res = []
    for cid, si in ((2, 0), (3, 0), (3, 1), (3, 2)):
        for r in (0.0, rate):
            p = workloads.make_problem(cid, si)
            sh = p.shape
            if r > 0:
                p.packed = workloads.draw_block_sparse_packed(workloads.rng_for(cid, 50, si), sh.N, sh.K, r,
                                                              workloads.CONFIGS[cid].code_probs)
            x, ws, ss, y, copies, _ = _device_problem(p, 1.0)
            maps = [tern.block_map(w) for w in ws]
            marked = float(np.unpackbits(maps[0].cpu().numpy().view(np.uint8)).sum()) / (sh.N * (sh.K // 128))
            t_dense = _graph_time_ms(lambda i: tern.matmul_into(x, ws[i % copies], ss[i % copies], y), 500, 10)
            t_skip = _graph_time_ms(lambda i: tern.matmul_blockmap_into(x, ws[i % copies], ss[i % copies],
                                                                        maps[i % copies], y), 500, 10)
            res.append({"workload": f"{workloads.CONFIGS[cid].name} M={sh.M} K={sh.K} N={sh.N}",
                        "zero_block_rate": r, "marked_fraction": round(marked, 4),
                        "dense_us": round(t_dense * 1e3, 3), "skip_us": round(t_skip * 1e3, 3),
                        "skip_over_dense": round(t_skip / t_dense, 4)})
            del x, ws, ss, y, maps
            torch.cuda.empty_cache()
    return res


def decode_sweep(reps: int = 3, fused: bool = False):
    """One token through 48 layers x 7 projections at M=1 (q, k, v, o 5120->5120; gate, up
    5120->17408; down 17408->5120): 336 launches over distinct weights captured in one graph.

    fused=True stores the projections that read the same activations as one matrix, as
    merged linear layers do (q|k|v: 5120->15360, gate|up: 5120->34816): the same weight
    bytes per token in 4 launches per layer (192) instead of 7."""
    import torch

    import ternary_weight_matmul_amd as tern
    import workloads

    dev = torch.device("cuda:0")
    cfg = workloads.CONFIGS[6]
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    xs = {k: torch.randn((1, k), generator=gen, device=dev).to(torch.bfloat16) for k in (5120, 17408)}
    shapes = [(sh.K, sh.N) for sh in cfg.shapes]
    if fused:
        layer = [(5120, 3 * 5120), (5120, 5120), (5120, 2 * 17408), (17408, 5120)]
        assert sorted(shapes[:7]) == sorted([(5120, 5120)] * 4 + [(5120, 17408)] * 2 + [(17408, 5120)])
        shapes = layer * (len(shapes) // 7)
    mats = []
    packed_bytes = scale_bytes = 0
    for K, N in shapes:
        w = workloads.draw_packed_device(gen, N, K, cfg.code_probs)
        s = workloads.draw_scales_device(gen, N, K // 128, cfg.scale_lo, cfg.scale_hi)
        y = torch.empty((1, N), dtype=torch.bfloat16, device=dev)
        mats.append((xs[K], w, s, y))
        packed_bytes += w.numel()
        scale_bytes += s.numel() * 2
    n = len(mats)
    ms = _graph_time_ms(lambda i: tern.matmul_into(*mats[i % n]), n * reps, n) * n
    tok_s = 1e3 / ms
    what = ("48 layers x (q|k|v, o, gate|up, down)" if fused else "48 layers x 7 projections")
    return {"workload": f"decode sweep: {what}, M=1, bf16",
            "launches_per_token": n, "ms_per_token": round(ms, 4), "tokens_per_s": round(tok_s, 2),
            "packed_weight_bytes_per_token": int(packed_bytes), "scale_bytes_per_token": int(scale_bytes),
            "packed_GBps": round(packed_bytes / (ms / 1e3) / 1e9, 1),
            "alg_GBps": round((packed_bytes + scale_bytes) / (ms / 1e3) / 1e9, 1),
            "hbm_roofline_ms_per_token": round((packed_bytes + scale_bytes) / (HBM_PEAK_GBS * 1e9) * 1e3, 4),
            "launch_floor_ms_per_token": f"{n} x ~1.5 us (see calibration)"}


def main():
    args = parse()
    if args.calibrate:
        print(json.dumps(calibrate(args.steps)), flush=True)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the ternary matmul path is built and measured per GPU, with no collectives.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import ternary_weight_matmul_amd as tern
    import workloads

    cfg = workloads.CONFIGS[args.config]
    p = workloads.make_problem(args.config, args.shape)
    sh = p.shape
    dev = torch.device("cuda:0")
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}

    x = torch.from_numpy(p.x.view(np.int16)).to(dev).view(tdt[p.x_dtype])
    w0 = torch.from_numpy(p.packed).to(dev)
    s0 = torch.from_numpy(p.scales.view(np.int16)).to(dev).view(torch.float16)
    wbytes = w0.numel() + s0.numel() * 2
    copies = max(1, int(np.ceil(args.rotate_gb * 1e9 / wbytes)))
    ws = [w0] + [w0.clone() for _ in range(copies - 1)]
    ss = [s0] + [s0.clone() for _ in range(copies - 1)]
    y = torch.empty((sh.M, sh.N), dtype=tdt[p.y_dtype], device=dev)

    def step(i):
        tern.matmul_into(x, ws[i % copies], ss[i % copies], y, path=args.path)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    if args.eager:
        t_wall = time.perf_counter()
        start.record()
        for i in range(args.steps):
            step(args.warmup + i)
        end.record()
        torch.cuda.synchronize()
        t_wall = time.perf_counter() - t_wall
    else:
        # The K timed steps are captured once into a HIP graph (a decode loop's
        # launches, as a serving loop would replay them) and replayed once, so
        # host launch overhead stays out of the measurement.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(args.warmup + i)
        graph.replay()                      # untimed replay: first-touch effects
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        start.record()
        graph.replay()
        end.record()
        torch.cuda.synchronize()
        t_wall = time.perf_counter() - t_wall
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    sec = ms_step / 1e3

    packed_bytes = sh.N * sh.K / 4
    scale_bytes = sh.N * (sh.K // 128) * 2
    xb = 2
    yb = {"f32": 4, "bf16": 2, "f16": 2}[p.y_dtype]
    alg_bytes = packed_bytes + scale_bytes + sh.M * sh.K * xb + sh.M * sh.N * yb
    flops = 2.0 * sh.M * sh.N * sh.K
    decode = sh.M <= 16
    if decode:
        value, unit = packed_bytes / sec / 1e9, "GB/s"
        achieved = alg_bytes / sec / 1e9
        traffic = measured_traffic(f"{cfg.name} M={sh.M} K={sh.K} N={sh.N}") if args.path == "auto" else None
        roof = {"bound": "hbm", "achieved": round(achieved, 3), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "traffic_unit": "HBM bytes per launch (FETCH_SIZE+WRITE_SIZE, copy-scaled)",
                "achieved_basis": "algorithmic bytes per launch / time per launch"}
    else:
        value, unit = flops / sec / 1e12, "TFLOP/s"
        achieved = flops / sec / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None}

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.x_dtype,
        "data": "synthetic (seeded; no model weights or datasets)",
        "config": {"workload": f"{cfg.name}: M={sh.M} K={sh.K} N={sh.N} ({sh.label})",
                   "M": sh.M, "K": sh.K, "N": sh.N, "group": 128, "x_dtype": p.x_dtype,
                   "y_dtype": p.y_dtype, "path": args.path, "weight_copies": copies,
                   "rotated_bytes": int(copies * wbytes), "parallelism": "single GPU",
                   "launch": "eager" if args.eager else "hip_graph"},
        "roofline": roof,
        "packed_weight_bytes": int(packed_bytes),
        "algorithmic_bytes": int(alg_bytes),
        "tflops": round(flops / sec / 1e12, 4),
        "packed_GBps_frac_of_hbm_peak": round(packed_bytes / sec / 1e9 / HBM_PEAK_GBS, 4),
        "wall_s_timed_region": round(t_wall, 4),
    }
    if not args.no_extras:
        del ws, ss
        torch.cuda.empty_cache()
        out["comparison_route"] = [comparison_route(args.config, args.shape), comparison_route(4, 3)]
        out["decode_sweep"] = decode_sweep()
        out["decode_sweep_fused_layout"] = decode_sweep(fused=True)
        torch.cuda.empty_cache()
        out["int8_scales"] = int8_scale_variant()
        out["zero_block_skip"] = zero_block_skip()
        out["other_workloads"] = other_workloads((args.config, args.shape))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
