"""Benchmark of the ternary-weight matmul on one MI355X.

Default workload: 27B-class attention-projection decode, M=1, K=N=5120,
bf16 activations, 2-bit packed weights with one fp16 scale per 128 weights,
bf16 output.  One step = one tern_matmul call (the whole per-token hot path
of that projection: stream the packed weights and scales, decode, sign-select
accumulate, scale at block boundaries, reduce, round, store).

Timing protocol (every timed figure in the record):
  * the weights come in `copies` distinct device copies spanning >= 2 GB, so
    no launch finds its weights in the 256 MB last-level cache;
  * one HIP graph holds L = max(steps, copies) launches, launch i reading
    copy i % copies: every replay streams every copy, and no copy is read
    twice within 2 GB of traffic;
  * after W eager warm-up launches and one untimed replay, the graph is
    replayed `replays` times, each bracketed by HIP events on the stream the
    kernels run on; the figure is the median over replays of the time per
    launch.  The record states L, the replays and the bytes each timed
    replay streamed.

Prints ONE JSON line.  `value` is packed-weight GB/s for M <= 16 decode
configurations and TFLOP/s for batched ones, as the metric defines them.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import struct
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, vendor figure
METRIC = ("packed-weight GB/s & % HBM peak (M=1 GEMV); TFLOP/s & % MFMA peak (M≥256)")
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
# host code that picks the kernel and its launch shape: the ABI dispatch and
# each kernel file's shape rules, so every library source counts
DISPATCH_SOURCES = "ternary_weight_matmul_amd/csrc"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--replays", type=int, default=5, help="timed replays of the graph (median reported)")
    ap.add_argument("--config", type=int, default=2, help="workload id (workloads.CONFIGS)")
    ap.add_argument("--shape", type=int, default=0, help="shape index inside the workload")
    ap.add_argument("--path", default="auto", choices=["auto", "gemv", "mfma", "gemv_mfma", "gemv_fp4", "gemv_b16"])
    ap.add_argument("--rotate-gb", type=float, default=2.0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-calibration", action="store_true")
    ap.add_argument("--calibrate", action="store_true", help="print only the calibration record")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="run the calibration copy kernel on BYTES bytes 20 times (for counter scaling)")
    ap.add_argument("--record-traffic", nargs=5, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                          "COPY_WRITE_DIR", "COPY_BYTES"),
                    help="write profiles/traffic.json for this workload from rocprofv3 --pmc csv output")
    ap.add_argument("--profile-doc", default="", metavar="PATH",
                    help="with --record-traffic: the profiles/ summary that gives the counters' commands")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the comparison route, the other workloads and the decode sweeps")
    ap.add_argument("--eager", action="store_true",
                    help="launch each step from Python instead of replaying a captured HIP graph")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# Code-object hash of a kernel (the traffic figure's guard)

def _elf_sections(b: bytes, base: int = 0):
    shoff = struct.unpack_from("<Q", b, base + 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", b, base + 0x3A)
    secs = []
    for i in range(shnum):
        name, typ, flags, addr, off, size, link, info, align, entsize = struct.unpack_from(
            "<IIQQQQIIQQ", b, base + shoff + i * shentsize)
        secs.append(dict(name=name, type=typ, addr=addr, off=off, size=size, link=link, entsize=entsize))
    strtab = secs[shstrndx]
    for s in secs:
        o = base + strtab["off"] + s["name"]
        s["name"] = b[o:b.index(b"\0", o)].decode()
    return secs


def device_functions(lib_path: str) -> dict:
    """{mangled name: machine-code bytes} of every gfx950 function in the library's
    offload bundles (the device code objects of this build)."""
    b = open(lib_path, "rb").read()
    fat = next(s for s in _elf_sections(b) if s["name"] == ".hip_fatbin")
    region = b[fat["off"]:fat["off"] + fat["size"]]
    out = {}
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    pos = region.find(magic)
    while pos >= 0:
        n = struct.unpack_from("<Q", region, pos + 24)[0]
        q = pos + 32
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", region, q)
            triple = region[q + 24:q + 24 + tlen].decode()
            q += 24 + tlen
            if "gfx950" not in triple:
                continue
            co = region[pos + off:pos + off + size]
            secs = _elf_sections(co)
            symtab = next(s for s in secs if s["name"] == ".symtab")
            strtab = secs[symtab["link"]]
            for i in range(symtab["size"] // 24):
                st_name, st_info, st_other, st_shndx, st_value, st_size = struct.unpack_from(
                    "<IBBHQQ", co, symtab["off"] + 24 * i)
                if st_info & 0xF != 2 or st_size == 0:     # STT_FUNC with a body
                    continue
                o = strtab["off"] + st_name
                name = co[o:co.index(b"\0", o)].decode()
                sec = secs[st_shndx]
                start = sec["off"] + st_value - sec["addr"]
                out[name] = co[start:start + st_size]
        pos = region.find(magic, pos + 24)
    return out


def kernel_code_sha256(symbols) -> str:
    import ternary_weight_matmul_amd as tern

    funcs = device_functions(tern.library_path())
    h = hashlib.sha256()
    for s in sorted(symbols):
        if s not in funcs:
            return ""
        h.update(s.encode())
        h.update(funcs[s])
    return h.hexdigest()


def dispatch_sha256() -> str:
    """SHA-256 over the library's sources (names and contents, sorted): a change to
    which kernel a shape gets, or to its launch shape, changes it."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, DISPATCH_SOURCES)
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode() + b"\0")
            h.update(open(os.path.join(d, name), "rb").read())
    return h.hexdigest()


def measured_traffic(workload_key: str):
    """HBM bytes per launch from profiles/traffic.json, if it still describes the built
    library: the machine code of the profiled kernel (hashed from the library's code
    object) and the library sources that choose the kernel and its launch shape must be
    the ones the counters were taken on."""
    try:
        entry = json.load(open(TRAFFIC_JSON))[workload_key]
    except (OSError, KeyError, ValueError):
        return None, "no counter record for this workload"
    if "kernel_symbols" not in entry or "dispatch_sha256" not in entry:
        return None, "counter record without the machine-code guard"
    if kernel_code_sha256(entry["kernel_symbols"]) != entry["kernel_code_sha256"]:
        return None, "kernel machine code changed since the counters were taken"
    if dispatch_sha256() != entry["dispatch_sha256"]:
        return None, "library sources (kernel choice or launch shape) changed since the counters were taken"
    return int(entry["hbm_bytes_per_launch"]), entry["profile"]


def _pmc_average(d: str, pattern: str):
    """Average per dispatch of each counter over the dispatches whose kernel name holds pattern."""
    import csv
    import glob

    vals, names = {}, set()
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if pattern in row.get("Kernel_Name", ""):
                vals.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
                names.add(row["Kernel_Name"])
    return {k: sum(v) / len(v) for k, v in vals.items()}, sorted(names)


def _dominant_kernel(d: str) -> str:
    """Base name (e.g. gemv_fp4_kernel) of the library kernel with the most dispatches in a
    rocprofv3 --pmc output directory."""
    import csv
    import glob
    import re

    count = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            m = re.search(r"tern::(?:\(anonymous namespace\)::)?(\w+_kernel)", row.get("Kernel_Name", ""))
            if m and m.group(1) != "stream_kernel":
                count[m.group(1)] = count.get(m.group(1), 0) + 1
    if not count:
        raise SystemExit(f"no library kernel in {d}")
    return max(count, key=count.get)


def record_traffic(args):
    """Write this workload's HBM bytes per launch into profiles/traffic.json, from four
    rocprofv3 --pmc runs: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the workload's
    kernel, and of the calibration copy of COPY_BYTES bytes (which scales each counter)."""
    import workloads

    fetch_dir, write_dir, cfetch_dir, cwrite_dir, copy_bytes = args.record_traffic
    copy_bytes = int(copy_bytes)
    cfg = workloads.CONFIGS[args.config]
    sh = cfg.shapes[args.shape]
    key = f"{cfg.name} M={sh.M} K={sh.K} N={sh.N}"
    pat = _dominant_kernel(fetch_dir) if args.path == "auto" else args.path
    f, fnames = _pmc_average(fetch_dir, pat)
    w, _ = _pmc_average(write_dir, pat)
    cf, _ = _pmc_average(cfetch_dir, "stream_kernel")
    cw, _ = _pmc_average(cwrite_dir, "stream_kernel")
    fscale = copy_bytes / (cf["FETCH_SIZE"] * 1024.0)
    wscale = copy_bytes / (cw["WRITE_SIZE"] * 1024.0)
    hbm = f["FETCH_SIZE"] * 1024.0 * fscale + w["WRITE_SIZE"] * 1024.0 * wscale
    funcs = device_functions(__import__("ternary_weight_matmul_amd").library_path())
    # the profiled kernel's mangled symbol: the device function whose demangled
    # template arguments appear in the profiled name
    syms = sorted(s for s in funcs if pat in s and any(_template_args(s) in n for n in fnames))
    try:
        data = json.load(open(TRAFFIC_JSON))
    except (OSError, ValueError):
        data = {}
    data[key] = {"workload": key, "kernel_names": fnames, "kernel_symbols": syms,
                 "kernel_code_sha256": kernel_code_sha256(syms), "dispatch_sha256": dispatch_sha256(),
                 "fetch_kib_per_dispatch": round(f["FETCH_SIZE"], 2), "write_kib_per_dispatch": round(w["WRITE_SIZE"], 2),
                 "copy_bytes": copy_bytes, "fetch_scale_from_copy": round(fscale, 5),
                 "write_scale_from_copy": round(wscale, 5), "hbm_bytes_per_launch": int(round(hbm)),
                 "profile": args.profile_doc or f"profiles/{key.split()[0]}_traffic.md"}
    json.dump(data, open(TRAFFIC_JSON, "w"), indent=1)
    print(json.dumps(data[key]))


def _template_args(mangled: str) -> str:
    """'<1, false, 5, 1>' for a mangled gemv_fp4_kernel<1, false, 5, 1> symbol."""
    import re

    i = mangled.index("I", mangled.index("kernel"))
    seg = mangled[i + 1:mangled.index("EE", i) + 1]
    vals = [("true" if v == "1" else "false") if k == "b" else v for k, v in re.findall(r"L([ib])(\d+)E", seg)]
    return "<" + ", ".join(vals) + ">"


# ---------------------------------------------------------------------------
# Timing

def timed_graph(launch, copies: int, steps: int, warmup: int, replays: int):
    """Median time per launch (ms) of a graph of L = max(steps, copies) launches, launch i
    reading copy i % copies; returns (median_ms, per-replay ms per launch, L)."""
    import numpy as np
    import torch

    L = max(steps, copies)
    for i in range(warmup):
        launch(L + i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(L):
            launch(i)
    g.replay()                       # untimed: first replay
    torch.cuda.synchronize()
    per = []
    for _ in range(replays):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) / L)
    del g
    return float(np.median(per)), per, L


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


def _graph_time_ms(step, copies, steps, warmup, replays=3):
    """Median ms per launch under the timing protocol (copies: the rotation period)."""
    return timed_graph(step, copies, steps, warmup, replays)[0]


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


# ---------------------------------------------------------------------------
# Calibration: launch floor and plain-read / copy ceilings (library kernel)

def calibration(sizes, replays: int = 5):
    """The plain streaming read of tern_stream_copy at each size (bytes), and a 1 GB copy,
    under the same protocol; plus the per-launch floor (a 16-byte read, one workgroup)."""
    import torch

    import ternary_weight_matmul_amd as tern

    dev = torch.device("cuda:0")
    region = 2_200_000_000
    buf = torch.empty(region, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    out = {"kernel": "tern_stream_copy: 512 threads x 4 loads of 16 B per workgroup, non-temporal"}
    tiny = buf[:16]
    floor_ms = _graph_time_ms(lambda i: tern.stream_copy(tiny), 1, 2000, 20, replays)
    out["launch_floor_us"] = round(floor_ms * 1e3, 3)
    reads = []
    for nbytes in sizes:
        nb = (int(nbytes) + 4095) // 4096 * 4096
        copies = max(1, (region - nb) // nb)
        views = [buf[i * nb:(i + 1) * nb] for i in range(copies)]
        ms = _graph_time_ms(lambda i: tern.stream_copy(views[i % copies]), copies, max(copies, 200), 5, replays)
        reads.append({"bytes": nb, "us": round(ms * 1e3, 3), "GBps": round(nb / (ms / 1e3) / 1e9, 1),
                      "frac_of_8TBps": round(nb / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)})
    out["stream_read"] = reads
    nb = 1 << 30
    src, dst = buf[:nb], buf[nb:2 * nb]
    ms = _graph_time_ms(lambda i: tern.stream_copy(src, dst), 1, 10, 2, replays)
    out["copy_1GiB"] = {"us": round(ms * 1e3, 1), "read_plus_write_GBps": round(2 * nb / (ms / 1e3) / 1e9, 1)}
    del buf
    torch.cuda.empty_cache()
    return out


def copy_probe(nbytes: int):
    import torch

    import ternary_weight_matmul_amd as tern

    buf = torch.empty(2 * nbytes, dtype=torch.uint8, device=torch.device("cuda:0"))
    buf.fill_(1)
    for _ in range(20):
        tern.stream_copy(buf[:nbytes], buf[nbytes:])
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "launches": 20}))


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on the host cores

def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(p, seconds: float, y_gpu):
    """The CPU oracle, as it stands, on bounded samples of the same workload: all threads
    (up to the box's 16-core share), then one thread; and the GPU result's largest
    error on the sampled outputs as a fraction of the allowed error."""
    import numpy as np

    import oracle

    o = oracle.default()
    sh = p.shape
    cores_avail = len(os.sched_getaffinity(0))
    threads = max(1, min(16, cores_avail))
    n_cols = sh.N if sh.M * sh.K * sh.N <= 3e8 else max(threads, int(3e8 // (sh.M * sh.K)))
    n_cols = min(n_cols, sh.N)

    def timed(ncols, nthreads, budget):
        reps, t0 = 0, time.perf_counter()
        Y = B = None
        while True:
            Y, B = o.matmul(p.x, p.x_dtype, p.packed[:ncols], p.scales[:ncols], sh.M, ncols, sh.K, threads=nthreads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return el / reps, reps, el, Y, B

    per, reps, el, Y, B = timed(n_cols, threads, seconds)
    n1 = max(1, n_cols // 16)
    per1, reps1, el1, _, _ = timed(n1, 1, max(1.0, seconds / 3))

    def rate(ncols, t):
        if sh.M == 1:
            return ncols * sh.K / 4 / t / 1e9
        return 2.0 * sh.M * ncols * sh.K / t / 1e12

    unit = "GB/s" if sh.M == 1 else "TFLOP/s"
    got = o.decode(y_gpu[:, :n_cols], p.y_dtype)
    ratio = float(np.max(np.abs(got - Y) / o.tolerance(Y, B, p.y_dtype)))
    return {"value": round(rate(n_cols, per), 6), "unit": unit, "cores": threads, "kind": "oracle",
            "sample": (f"{reps} full oracle passes over {n_cols} of {sh.N} output columns "
                       f"(M={sh.M}, K={sh.K}) on {threads} threads, {el:.1f} s"),
            "threads": threads, "host_cpus_in_affinity": cores_avail, "cpu_model": _cpu_model(),
            "value_1_thread": round(rate(n1, per1), 6),
            "sample_1_thread": f"{reps1} passes over {n1} columns on 1 thread, {el1:.1f} s",
            "gpu_max_err_over_allowance": round(ratio, 4),
            "allowance": "2e-3 * sum_k |x s| + one ulp of the output type, on the sampled columns"}


# ---------------------------------------------------------------------------
# Extras (same protocol, fewer launches)

def other_workloads(skip, replays):
    """Every configured shape except the headline one."""
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
            ms = _graph_time_ms(lambda i: tern.matmul_into(x, ws[i % copies], ss[i % copies], y), copies, steps, 5,
                                replays)
            res.append({"workload": f"{workloads.CONFIGS[cid].name} ({sh.label})", **_summary(p, ms)})
            del x, ws, ss, y
            torch.cuda.empty_cache()
    return res


def comparison_route(cid, si, replays):
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
    t_deq = _graph_time_ms(lambda i: tern.dequant(w, s, out=W), 1, steps, 5, replays)
    t_gemm = _graph_time_ms(lambda i: torch.matmul(W, xT, out=yT), 1, steps, 5, replays)
    t_fused = _graph_time_ms(lambda i: tern.matmul_into(x, w, s, y), 1, steps, 5, replays)
    return {"workload": f"{workloads.CONFIGS[cid].name} M={sh.M} K={sh.K} N={sh.N}",
            "dequant_us": round(t_deq * 1e3, 3), "library_gemm_us": round(t_gemm * 1e3, 3),
            "route_total_us": round((t_deq + t_gemm) * 1e3, 3), "fused_us": round(t_fused * 1e3, 3),
            "route_over_fused": round((t_deq + t_gemm) / t_fused, 3),
            "dense_weight_bytes": int(sh.N * sh.K * 2), "packed_weight_bytes": int(sh.N * sh.K // 4),
            "note": "weights resident (no rotation) for both routes"}


def int8_scale_variant(replays):
    """fp16 block scales vs int8 codes with a per-row fp32 factor (tern_matmul_s8) on the
    decode and batched shapes (weights rotated over 1 GB)."""
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
        t16 = _graph_time_ms(lambda i: tern.matmul_into(x, ws[i % copies], ss[i % copies], y), copies, steps, 5,
                             replays)
        t8 = _graph_time_ms(lambda i: tern.matmul_s8_into(x, ws[i % copies], qr[i % copies][0],
                                                          qr[i % copies][1], y), copies, steps, 5, replays)
        packed = sh.N * sh.K // 4
        res.append({"workload": f"{workloads.CONFIGS[cid].name} M={sh.M} K={sh.K} N={sh.N}",
                    "fp16_scales_us": round(t16 * 1e3, 3), "int8_scales_us": round(t8 * 1e3, 3),
                    "int8_over_fp16": round(t8 / t16, 4),
                    "weight_bytes_fp16_scales": int(packed + sh.N * (sh.K // 128) * 2),
                    "weight_bytes_int8_scales": int(packed + sh.N * (sh.K // 128) + 4 * sh.N)})
        del x, ws, ss, y, qr
        torch.cuda.empty_cache()
    return res


def zero_block_skip(replays, rate: float = 0.5):
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
            t_dense = _graph_time_ms(lambda i: tern.matmul_into(x, ws[i % copies], ss[i % copies], y), copies,
                                     500, 5, replays)
            t_skip = _graph_time_ms(lambda i: tern.matmul_blockmap_into(x, ws[i % copies], ss[i % copies],
                                                                        maps[i % copies], y), copies, 500, 5,
                                    replays)
            res.append({"workload": f"{workloads.CONFIGS[cid].name} M={sh.M} K={sh.K} N={sh.N}",
                        "zero_block_rate": r, "marked_fraction": round(marked, 4),
                        "dense_us": round(t_dense * 1e3, 3), "skip_us": round(t_skip * 1e3, 3),
                        "skip_over_dense": round(t_skip / t_dense, 4)})
            del x, ws, ss, y, maps
            torch.cuda.empty_cache()
    return res


def decode_sweep(replays, fused: bool = False):
    """One token through 48 layers x 7 projections at M=1 (q, k, v, o 5120->5120; gate, up
    5120->17408; down 17408->5120): 336 launches over distinct weights (4.47 GB) per
    graph replay.

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
    ms = _graph_time_ms(lambda i: tern.matmul_into(*mats[i % n]), n, n, n, replays) * n
    tok_s = 1e3 / ms
    what = ("48 layers x (q|k|v, o, gate|up, down)" if fused else "48 layers x 7 projections")
    return {"workload": f"decode sweep: {what}, M=1, bf16",
            "launches_per_token": n, "ms_per_token": round(ms, 4), "tokens_per_s": round(tok_s, 2),
            "packed_weight_bytes_per_token": int(packed_bytes), "scale_bytes_per_token": int(scale_bytes),
            "packed_GBps": round(packed_bytes / (ms / 1e3) / 1e9, 1),
            "alg_GBps": round((packed_bytes + scale_bytes) / (ms / 1e3) / 1e9, 1),
            "hbm_roofline_ms_per_token": round((packed_bytes + scale_bytes) / (HBM_PEAK_GBS * 1e9) * 1e3, 4)}


# ---------------------------------------------------------------------------

def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the ternary matmul path is built and measured per GPU, with no collectives.",
              file=sys.stderr)
        sys.exit(2)
    if args.record_traffic:
        record_traffic(args)
        return
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    import numpy as np
    import torch

    import ternary_weight_matmul_amd as tern
    import workloads

    cfg = workloads.CONFIGS[args.config]
    p = workloads.make_problem(args.config, args.shape)
    sh = p.shape
    packed_bytes = sh.N * sh.K / 4
    scale_bytes = sh.N * (sh.K // 128) * 2
    yb = {"f32": 4, "bf16": 2, "f16": 2}[p.y_dtype]
    alg_bytes = packed_bytes + scale_bytes + sh.M * sh.K * 2 + sh.M * sh.N * yb
    if args.calibrate:
        print(json.dumps({"calibration": calibration([alg_bytes, 23.7e6, 1 << 30], args.replays)}), flush=True)
        return

    x, ws, ss, y, copies, wbytes = _device_problem(p, args.rotate_gb)

    def step(i):
        tern.matmul_into(x, ws[i % copies], ss[i % copies], y, path=args.path)

    t_wall = time.perf_counter()
    if args.eager:
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_wall = time.perf_counter()
        start.record()
        for i in range(args.steps):
            step(args.warmup + i)
        end.record()
        torch.cuda.synchronize()
        ms_step, per, L = start.elapsed_time(end) / args.steps, [], args.steps
    else:
        ms_step, per, L = timed_graph(step, copies, args.steps, args.warmup, args.replays)
    t_wall = time.perf_counter() - t_wall
    sec = ms_step / 1e3
    y_gpu = out_bits(y, p.y_dtype)

    flops = 2.0 * sh.M * sh.N * sh.K
    decode = sh.M <= 16
    if decode:
        value, unit = packed_bytes / sec / 1e9, "GB/s"
        achieved = alg_bytes / sec / 1e9
        traffic, traffic_src = (measured_traffic(f"{cfg.name} M={sh.M} K={sh.K} N={sh.N}")
                                if args.path == "auto" else (None, "forced path"))
        roof = {"bound": "hbm", "achieved": round(achieved, 3), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, each scaled by a copy of known size)",
                "traffic_source": traffic_src,
                "achieved_basis": "algorithmic bytes per launch / median time per launch"}
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
                   "weight_bytes_per_copy": int(wbytes),
                   "rotated_bytes": int(L * wbytes) if not args.eager else int(args.steps * wbytes),
                   "parallelism": "single GPU", "launch": "eager" if args.eager else "hip_graph"},
        "timing": {"launches_per_replay": L, "timed_replays": len(per),
                   "us_per_launch_each_replay": [round(v * 1e3, 4) for v in per],
                   "statistic": "median over replays of time per launch" if per else "mean over eager launches",
                   "bytes_streamed_per_timed_replay": int(L * wbytes) if per else None},
        "roofline": roof,
        "packed_weight_bytes": int(packed_bytes),
        "algorithmic_bytes": int(alg_bytes),
        "tflops": round(flops / sec / 1e12, 4),
        "packed_GBps_frac_of_hbm_peak": round(packed_bytes / sec / 1e9 / HBM_PEAK_GBS, 4),
        "wall_s_timed_region": round(t_wall, 4),
    }
    del ws, ss
    torch.cuda.empty_cache()
    if not args.no_calibration:
        out["calibration"] = calibration([alg_bytes, 23.7e6, 1 << 30], args.replays)
    if not args.no_extras:
        out["comparison_route"] = [comparison_route(args.config, args.shape, 3), comparison_route(4, 3, 3)]
        out["decode_sweep"] = decode_sweep(3)
        out["decode_sweep_fused_layout"] = decode_sweep(3, fused=True)
        torch.cuda.empty_cache()
        out["int8_scales"] = int8_scale_variant(3)
        out["zero_block_skip"] = zero_block_skip(3)
        out["other_workloads"] = other_workloads((args.config, args.shape), 3)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds, y_gpu)
    print(json.dumps(out), flush=True)


def out_bits(y, y_dtype):
    """The output tensor's bits as numpy (uint16 for 16-bit types, float32 otherwise)."""
    import numpy as np
    import torch

    if y_dtype == "f32":
        return y.float().cpu().numpy()
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


if __name__ == "__main__":
    main()
