"""Builds libxhc.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m residual_stream_architecture_amd.build
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["xhc_api.cpp", "xhc_fwd.hip", "xhc_bwd.hip", "xhc_chain.hip", "xhc_route.hip", "xhc_noalloc.hip"]
LIB = os.path.join(PKG, "libxhc.so")
# bandwidth probes for the benchmark: a library of their own, not part of libxhc
PROBE_SOURCE = "xhc_probe.hip"
PROBE_LIB = os.path.join(PKG, "libxhc_probe.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # keep the compiler from emitting packed fp32 math (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the 12-token sliding-window loops are unrolled in full so that the
    # window index stays a compile-time register index
    "-mllvm", "-pragma-unroll-threshold=100000",
    "-Wno-unused-result",
    "-I" + os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objs = []
    cmds = []
    for s in SOURCES + [PROBE_SOURCE]:
        obj = os.path.join(BUILD_DIR, s + ".o")
        objs.append(obj)
        cmds.append([hipcc, *FLAGS, "-c", os.path.join(CSRC, s), "-o", obj])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    for lib, lib_objs in ((LIB, objs[:-1]), (PROBE_LIB, objs[-1:])):
        tmp = lib + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *lib_objs])
        _check_kernel_stubs(tmp)
        os.replace(tmp, lib)
    return LIB


def _check_kernel_stubs(lib):
    """A kernel template whose host-side instantiation fails (a deferred
    device-code diagnostic) leaves its launch stub undefined: the library
    links but cannot be loaded.  Fail the build instead."""
    try:
        out = subprocess.run(["nm", "-D", "--undefined-only", lib], stdout=subprocess.PIPE,
                             stderr=subprocess.DEVNULL, text=True).stdout
    except FileNotFoundError:
        return
    missing = [l.split()[-1] for l in out.splitlines() if "__device_stub__" in l]
    if missing:
        os.remove(lib)
        raise RuntimeError("kernel launch stubs missing from the library (host-side instantiation failed):\n  "
                           + "\n  ".join(missing))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
