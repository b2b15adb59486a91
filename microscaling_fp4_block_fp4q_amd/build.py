"""Build libfp4q.so (HIP, gfx950) in-tree.

    python -m microscaling_fp4_block_fp4q_amd.build

Each csrc/*.hip translation unit is compiled by its own hipcc process (in
parallel), then linked into microscaling_fp4_block_fp4q_amd/libfp4q.so.
The measurement probes of the benchmark (probe/*.hip: HBM streams and VALU
issue rates, not part of the path) become libfp4q_probe.so.

Floating-point flags are part of the numerical contract: no FMA
contraction, correctly rounded fp32 division, fp32 denormals kept, no
fast-math; packed fp32 instructions are disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfp4q.so")
PROBE = os.path.join(PKG, "probe")
PROBE_LIB = os.path.join(PKG, "libfp4q_probe.so")

ARCH = os.environ.get("FP4Q_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++20",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def sources(folder: str = CSRC) -> list[str]:
    return sorted(os.path.join(folder, f) for f in os.listdir(folder) if f.endswith(".hip"))


def _compile(src: str) -> str:
    prefix = "probe_" if os.path.dirname(src) == PROBE else ""
    obj = os.path.join(BUILD, prefix + os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every translation unit, link libfp4q.so and the benchmark's
    probe library; returns the path of libfp4q.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    probe_srcs = sources(PROBE)
    jobs = jobs or min(len(srcs) + len(probe_srcs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs + probe_srcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
