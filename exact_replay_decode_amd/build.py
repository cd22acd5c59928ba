"""Build libssd_replay.so (HIP, gfx950) in-tree with hipcc.

    python -m exact_replay_decode_amd.build

-ffp-contract=off: every fused multiply-add in the kernels is an explicit
fmaf, so the prefill and decode kernels round identically. Packed fp32
instructions are switched off for the device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libssd_replay.so")
# the bench's bandwidth probe, a separate library (not part of the scan)
PROBE_LIB = os.path.join(HERE, "libssd_probe.so")
PROBE_SOURCE = "ssd_probe.hip"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["ssd_api.cpp", "ssd_scalar.hip", "ssd_mfma.hip", "ssd_conv.hip", "ssd_scratch.hip"]
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form"]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


OBJDIR = os.path.join(HERE, "_build")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math", "-Wall",
          "-I", INCLUDE, "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in r.stderr.splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)


def build(verbose: bool = False) -> str:
    """Compile every source (one hipcc process per file, in parallel), then
    link the shared library."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(OBJDIR, exist_ok=True)
    objs = [os.path.join(OBJDIR, os.path.basename(src) + ".o") for src in sources()]
    cmds = [[HIPCC, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, "-x", "hip", "-c", src,
             "-o", obj] for src, obj in zip(sources(), objs)]
    with ThreadPoolExecutor(len(cmds)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, "-shared", "-x", "hip",
          os.path.join(CSRC, PROBE_SOURCE), "-o", tmp], verbose)
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
