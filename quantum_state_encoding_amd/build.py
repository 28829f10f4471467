"""Build libfwt.so (the HIP kernels and the C ABI) for gfx950, in-tree."""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfwt.so")
SOURCES = [os.path.join(CSRC, "fwt_kernels.hip"), os.path.join(CSRC, "fwt_ablation.hip"),
           os.path.join(CSRC, "fwt_ozaki.hip"), os.path.join(CSRC, "fwt_static.hip"),
           os.path.join(CSRC, "fwt_api.cpp")]
HEADERS = [os.path.join(CSRC, "fwt_internal.h"), os.path.join(ROOT, "include", "fwt.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions are disabled: the compiler would otherwise
# pair the float4 butterflies into v_pk_* forms.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def stale():
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


def build(force=True, verbose=False):
    """Compile the library; returns its path."""
    if not force and not stale():
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
