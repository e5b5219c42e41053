"""Build libve.so (gfx950) in-tree with hipcc.

    python -m ragged_shard_optimizer_amd.build
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "_build", "libve.so")
SOURCES = [os.path.join(CSRC, f) for f in ("ve_host.cpp", "ve_planner.cpp", "ve_muon_host.cpp", "ve_kernels.hip", "ve_group.hip",
                                           "ve_muon.hip", "ve_stream.hip",
                                           "ve_muon_static.hip")]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # fused multiply-adds only where written explicitly
    "-ffp-contract=off",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is expected
    noise = [ln for ln in (res.stderr or "").splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(noise))
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)


def build(verbose: bool = False, defines=()) -> str:
    """Compile every source to an object (in parallel), then link libve.so.
    ``defines``: extra ``NAME=VALUE`` macros (measurement builds)."""
    from concurrent.futures import ThreadPoolExecutor
    odir = os.path.join(os.path.dirname(OUT), f"obj{os.getpid()}")
    os.makedirs(odir, exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if f != "-shared"] + [f"-D{d}" for d in defines]
    objs = [os.path.join(odir, os.path.basename(src) + ".o") for src in SOURCES]
    jobs = min(len(SOURCES), max(1, os.cpu_count() or 1))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _run(["hipcc", *flags, "-c", so[0], "-o", so[1]], verbose), zip(SOURCES, objs)))
    tmp = OUT + f".tmp{os.getpid()}"
    _run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    for o in objs:
        os.remove(o)
    os.rmdir(odir)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
