"""Build libve.so (gfx950) in-tree with hipcc.

    python -m ragged_shard_optimizer_amd.build [--sanitize]

``--sanitize`` builds libve_san.so and the oracle's sanitized twin with
host-side AddressSanitizer and UBSan; the CPU test suite then runs against
them with

    VE_SANITIZED=1 ASAN_OPTIONS=detect_leaks=0 \
    LD_PRELOAD=$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so) \
    python -m pytest tests -m "not gpu" -p no:xdist
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


# Host-side AddressSanitizer + UBSan (device code is built as usual); the
# result is libve_san.so, loaded by the binding when VE_SANITIZED=1 and run
# with the clang ASan runtime preloaded (see the module docstring).
SAN_OUT = os.path.join(PKG, "_build", "libve_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined", "-g"]


def build(verbose: bool = False, defines=(), sanitize: bool = False) -> str:
    """Compile every source to an object (in parallel), then link libve.so
    (libve_san.so with ``sanitize``).  ``defines``: extra ``NAME=VALUE``
    macros (measurement builds)."""
    from concurrent.futures import ThreadPoolExecutor
    out = SAN_OUT if sanitize else OUT
    odir = os.path.join(os.path.dirname(OUT), f"obj{os.getpid()}")
    os.makedirs(odir, exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if f != "-shared"] + [f"-D{d}" for d in defines] + (SAN_FLAGS if sanitize else [])
    objs = [os.path.join(odir, os.path.basename(src) + ".o") for src in SOURCES]
    jobs = min(len(SOURCES), max(1, os.cpu_count() or 1))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _run(["hipcc", *flags, "-c", so[0], "-o", so[1]], verbose), zip(SOURCES, objs)))
    tmp = out + f".tmp{os.getpid()}"
    link = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"] if sanitize else []
    _run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *link, *objs, "-o", tmp], verbose)
    for o in objs:
        os.remove(o)
    os.rmdir(odir)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        sys.path.insert(0, ROOT)
        import oracle
        print(oracle.build(force=True, sanitize=True))
        print(build(verbose=True, sanitize=True))
    else:
        print(build(verbose=True))
