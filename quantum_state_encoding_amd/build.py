"""Build libfwt.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Each source compiles to its own object (in parallel, under _build/), then
one link makes the library.  build(force=True) recompiles every source;
build(force=False) recompiles only objects older than their source or any
header."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfwt.so")
OBJDIR = os.path.join(PKG, "_build")
SOURCES = [os.path.join(CSRC, f) for f in ("fwt_kernels.hip", "fwt_onepass.hip",
                                           "fwt_ablation.hip", "fwt_ozaki.hip",
                                           "fwt_static.hip", "fwt_api.cpp")]
HEADERS = [os.path.join(CSRC, "fwt_internal.h"), os.path.join(CSRC, "fwt_device.h"),
           os.path.join(ROOT, "include", "fwt.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions are disabled: the compiler would otherwise
# pair the float4 butterflies into v_pk_* forms.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
         "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _obj(src):
    return os.path.join(OBJDIR, os.path.basename(src) + ".o")


def _stale_obj(src):
    o = _obj(src)
    if not os.path.exists(o):
        return True
    t = os.path.getmtime(o)
    return any(os.path.getmtime(f) > t for f in [src] + HEADERS)


def stale():
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)


def build(force=True, verbose=False):
    """Compile the library; returns its path."""
    if not force and not stale():
        return LIB
    os.makedirs(OBJDIR, exist_ok=True)
    todo = [s for s in SOURCES if force or _stale_obj(s)]
    jobs = max(1, min(len(todo), len(os.sched_getaffinity(0)), 6))
    with ThreadPoolExecutor(jobs) as ex:
        for f in [ex.submit(_run, [HIPCC] + FLAGS + ["-c", s, "-o", _obj(s)], verbose)
                  for s in todo]:
            f.result()
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + [_obj(s) for s in SOURCES] +
         ["-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
