"""Build libar.so (HIP kernels + C ABI) in-tree for gfx950.

Run ``python ring_allreduce_rs_amd/_build.py`` or ``__graft_entry__.build()``
(the script does not import the package, which needs the library).
hipcc cross-compiles for gfx950 without a GPU present.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libar.so")

# the fused kernels are instantiated per element type so the (slowest) device
# compilations run side by side
SOURCES = ["fused_f32.hip", "fused_f32_lead.hip", "fused_bf16.hip", "fused_bf16_lead.hip",
           "fused_i32.hip", "fused_i32_lead.hip", "fused.hip", "steps.hip", "copy.hip",
           "check.hip", "probe.hip", "dispatch.hip", "ar_api.cpp"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # exact per-hop arithmetic: no contraction, IEEE division, subnormals kept
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # never form packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libar.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}: {' '.join(cmd[-3:])}")
    if verbose and res.stderr.strip():
        sys.stderr.write(res.stderr)


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source (in parallel) and link ring_allreduce_rs_amd/libar.so;
    returns its path."""
    flags = [*FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC]
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1)), 16))
    with tempfile.TemporaryDirectory(prefix="ar_build_") as tmpdir:
        objs = [os.path.join(tmpdir, s + ".o") for s in SOURCES]
        cmds = [[hipcc(), *flags, "-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=jobs) as pool:
            for f in [pool.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = LIB + ".tmp"
        _run([hipcc(), *FLAGS, *(extra_flags or []), "-shared", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, extra_flags=sys.argv[1:]))
