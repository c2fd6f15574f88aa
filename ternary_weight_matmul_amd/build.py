"""Build libtern.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "libtern.so")
ARCH = os.environ.get("TERN_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set ROCM_PATH)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(out: str = LIBRARY, verbose: bool = False) -> str:
    """Compile every csrc/*.hip into one shared library; always recompiles."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           # packed-fp32 VALU forms are kept out of every kernel
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument",
           "-o", tmp] + sources()
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass warns that it does not know the device-only feature; keep other output
    lines = [l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l]
    if res.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError("hipcc failed (exit %d)" % res.returncode)
    if verbose and lines:
        print("\n".join(lines))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
