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


SAN_DIR = os.path.join(BUILD_DIR, "san")
SAN_LIB = os.path.join(SAN_DIR, "libxhc.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def build_sanitized():
    """libxhc.so with its C-ABI layer (validation, planning, dispatch, timer:
    xhc_api.cpp) compiled as plain host C++ under AddressSanitizer and
    UBSan, linked with the kernels' objects of build(), into _build/san.
    For the ABI tests on the CPU: load it with XHC_LIBRARY and the ASan
    runtime preloaded (sanitized_env())."""
    if not all(os.path.exists(os.path.join(BUILD_DIR, s + ".o")) for s in SOURCES[1:]):
        build()
    os.makedirs(SAN_DIR, exist_ok=True)
    api_obj = os.path.join(SAN_DIR, "xhc_api.o")
    _run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I" + os.path.join(ROOT, "include"), "-Wno-unused-result", *SAN_FLAGS,
          "-c", os.path.join(CSRC, SOURCES[0]), "-o", api_obj])
    objs = [os.path.join(BUILD_DIR, s + ".o") for s in SOURCES[1:]]
    _run(["g++", "-shared", *SAN_FLAGS, "-o", SAN_LIB, api_obj, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib"])
    return SAN_LIB


def sanitized_env():
    """Environment that loads SAN_LIB in a Python process (the interpreter
    itself is not instrumented, so the ASan runtime is preloaded)."""
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], stdout=subprocess.PIPE, text=True).stdout.strip()
    env = dict(os.environ)
    env.update(XHC_LIBRARY=SAN_LIB, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


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
