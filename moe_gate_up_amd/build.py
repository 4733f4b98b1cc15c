"""Build the HIP library libmoe_decode.so in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libmoe_decode.so")
BUILD_DIR = os.path.join(HERE, "_build")

# Translation units and their own flags.  The two down kernel families take
# other instruction-scheduling strategies than the rest of the library (why,
# with the measurements, in csrc/host.hpp).
SOURCES = [
    ("moe_decode.hip", []),
    ("down_token.hip", ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"]),
    ("down_mfma.hip", ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]),
]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-FP32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernel arguments preloaded into SGPRs when the wave starts: one scalar
    # load round trip less before a kernel's first (dependent) loads; at one
    # token per step that is 2 % of the layer (12.4 -> 12.1 us on MI355X)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall",
]


def hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if p and (os.path.sep not in p or os.path.exists(p)):
            return p
    return "hipcc"


def _run(cmds, verbose):
    """Run the commands in parallel; raise with the first failure's messages."""
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    failed = None
    for p in procs:
        _, stderr = p.communicate()
        err = "\n".join(l for l in stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
        if p.returncode != 0 and failed is None:
            failed = f"hipcc failed ({p.returncode}):\n{err}"
        elif err and verbose:
            print(err, file=sys.stderr)
    if failed:
        raise RuntimeError(failed)


def build(out: str = OUT, verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    objs, cmds = [], []
    for src, extra in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc(), *HIPCC_FLAGS, *extra, *inc, "-c", os.path.join(HERE, "csrc", src), "-o", obj])
    _run(cmds, verbose)
    _run([[hipcc(), "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", out + ".tmp"]], verbose)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
