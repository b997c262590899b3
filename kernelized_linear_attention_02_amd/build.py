"""Build libkla.so for gfx950 with hipcc, in-tree, next to this file.

Every HIP source under csrc/ is compiled to an object, then linked into one
shared library that exports the C ABI of include/kla.h.
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkla.so")

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from emitting packed fp32 ALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-fvisibility=hidden",
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; ROCm is required to build libkla")
    return p


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def kernel_resources(stderr: str):
    """Per-kernel resource remarks: {kernel: {"ScratchSize": n, "VGPRs": n, ...}}."""
    out, cur = {}, None
    for line in stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+) \[-Rpass", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return out


def _compile(src: str, verbose: bool):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, "-Rpass-analysis=kernel-resource-usage",
           "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    res = kernel_resources(r.stderr)
    if verbose:
        # the host pass warns about the packed-fp32 target feature; keep other warnings visible
        lines = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and "remark" not in l
                 and not l.startswith(" ")]
        if any(l.strip() for l in lines):
            print("\n".join(lines), file=sys.stderr)
    return obj, res


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(8, len(srcs))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), srcs))
    objs = [o for o, _ in results]
    # Register spills are refused: besides their cost, spill code placed in
    # divergent regions has been seen to lose values on this toolchain.
    spills = {k: v for _, res in results for k, v in res.items()
              if v.get("ScratchSize", 0) > 0 or v.get("VGPRs Spill", 0) > 0}
    if spills:
        names = "\n  ".join(f"{k}: {v}" for k, v in sorted(spills.items()))
        raise RuntimeError(f"kernels use scratch memory (register spills):\n  {names}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
