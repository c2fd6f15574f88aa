"""Build libtern.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Each csrc/*.hip is compiled to its own object (in parallel, with any
per-file flags in PER_FILE), then the objects are linked into one shared
library.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "libtern.so")
ARCH = os.environ.get("TERN_OFFLOAD_ARCH", "gfx950")

COMMON = ["-O3", "-std=c++17", "-fPIC",
          # packed-fp32 VALU forms are kept out of every kernel
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]
PER_FILE = {}   # file name -> extra hipcc flags


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set ROCM_PATH)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass warns that it does not know the device-only feature; keep other output
    lines = [l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l]
    return res.returncode, lines


def build(out: str = LIBRARY, verbose: bool = False) -> str:
    """Compile every csrc/*.hip and link one shared library; always recompiles."""
    tag = "%d" % os.getpid()
    objdir = os.path.join(HERE, "_build_obj")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    jobs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src)[:-4] + "." + tag + ".o")
        cmd = [cc, "--offload-arch=" + ARCH, "-c"] + COMMON + PER_FILE.get(os.path.basename(src), []) + \
            ["-o", obj, src]
        jobs.append((src, obj, cmd))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda j: _run(j[2]), jobs))
    failed = False
    for (src, _, cmd), (rc, lines) in zip(jobs, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            failed = True
            sys.stderr.write("\n".join(lines) + "\n")
        elif verbose and lines:
            print("\n".join(lines))
    tmp = out + ".tmp" + tag
    try:
        if failed:
            raise RuntimeError("hipcc failed")
        link = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + [o for _, o, _ in jobs]
        if verbose:
            print(" ".join(link), flush=True)
        rc, lines = _run(link)
        if rc != 0:
            sys.stderr.write("\n".join(lines) + "\n")
            raise RuntimeError("link failed (exit %d)" % rc)
        os.replace(tmp, out)
    finally:
        for _, o, _ in jobs:
            if os.path.exists(o):
                os.remove(o)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
