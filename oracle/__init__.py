"""CPU oracle for the batched Walsh-Hadamard transform.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in
__graft_entry__ and the CPU-baseline leg of bench.py may import this
package.  The product path (quantum_state_encoding_amd) never imports,
loads or calls it, and the two share no code.

Two independent implementations of the same definition live here:

* ``liboracle.so`` (oracle.c): brute force from the entry definition, the
  textbook iterative butterfly network in fp64 ("check mode") and fp32
  (timed mode), and the Kronecker-composed form.
* ``brute_numpy``: the definition written with numpy's bitwise_count, used
  to pin the C code on small n.

Definition (per real vector x of length N = 2^n; re and im of a planar
complex state are transformed independently because the matrix is real):
y_k = c * sum_i (-1)^popcount(k & i) x_i, c = 1 or 2^(-n/2).  The entry is
the on-the-fly Walsh coefficient of the Apache Mahout pull request
"[QDP] [feature] Pr4 kronecker fwt", section "How".
"""
import ctypes
import os

import numpy as np

from .build import LIB, SRC, build_oracle

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build_oracle()
        lib = ctypes.CDLL(LIB)
        i64, i32 = ctypes.c_int64, ctypes.c_int
        pd = ctypes.POINTER(ctypes.c_double)
        pf = ctypes.POINTER(ctypes.c_float)
        lib.oracle_bruteforce_f64.argtypes = [pd, pd, i64, i32, i32]
        lib.oracle_bruteforce_f64.restype = None
        lib.oracle_fwt_f64.argtypes = [pd, i64, i32, i32]
        lib.oracle_fwt_f64.restype = None
        lib.oracle_fwt_f32.argtypes = [pf, i64, i32, i32]
        lib.oracle_fwt_f32.restype = None
        lib.oracle_fwt_kron_f64.argtypes = [pd, i64, i32, i32, i32]
        lib.oracle_fwt_kron_f64.restype = i32
        lib.oracle_fwt_threaded_f32.argtypes = [pf, i64, i32, i32, i32]
        lib.oracle_fwt_threaded_f32.restype = i32
        lib.oracle_fwt_threaded_f64.argtypes = [pd, i64, i32, i32, i32]
        lib.oracle_fwt_threaded_f64.restype = i32
        lib.oracle_fwt_ld.argtypes = [pd, pd, i64, i32, i32]
        lib.oracle_fwt_ld.restype = i32
        lib.oracle_norm_constant_f64.argtypes = [i32]
        lib.oracle_norm_constant_f64.restype = ctypes.c_double
        lib.oracle_norm_constant_f32.argtypes = [i32]
        lib.oracle_norm_constant_f32.restype = ctypes.c_float
        _lib = lib
    return _lib


def _as_rows(x, n, dtype):
    a = np.ascontiguousarray(x, dtype=dtype)
    N = 1 << n
    if a.size % N:
        raise ValueError("size %d is not a multiple of 2^%d" % (a.size, n))
    return a, a.size // N


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def norm_constant(n, dtype=np.float64):
    """c = 2^(-n/2) as the oracle applies it (rounded once to dtype)."""
    lib = _load()
    if np.dtype(dtype) == np.float32:
        return np.float32(lib.oracle_norm_constant_f32(n))
    return np.float64(lib.oracle_norm_constant_f64(n))


def fwt(x, n, normalize=False, dtype=np.float64):
    """Textbook iterative transform of every length-2^n row of x.

    Returns a new array of ``dtype`` (float64 = check mode, float32 = the
    timed-mode precision) with the input's shape.
    """
    a, nvec = _as_rows(x, n, dtype)
    a = a.copy()
    lib = _load()
    if a.dtype == np.float32:
        lib.oracle_fwt_f32(_ptr(a, ctypes.c_float), nvec, n, int(bool(normalize)))
    elif a.dtype == np.float64:
        lib.oracle_fwt_f64(_ptr(a, ctypes.c_double), nvec, n, int(bool(normalize)))
    else:
        raise TypeError("dtype must be float32 or float64")
    return a.reshape(np.shape(x))


def fwt_complex(re, im, n, normalize=False):
    """Planar complex state: the real and imaginary parts transformed
    independently, in fp64."""
    return fwt(re, n, normalize), fwt(im, n, normalize)


def bruteforce(x, n, normalize=False):
    """O(4^n) definition, fp64 accumulation (C implementation)."""
    a, nvec = _as_rows(x, n, np.float64)
    y = np.empty_like(a)
    _load().oracle_bruteforce_f64(_ptr(a, ctypes.c_double), _ptr(y, ctypes.c_double),
                                  nvec, n, int(bool(normalize)))
    return y.reshape(np.shape(x))


def fwt_ld(x, n, normalize=False):
    """The textbook transform evaluated in long double (64-bit significand on
    x86-64) and rounded to float64 once: a higher-precision cross-check of
    the fp64 check mode."""
    a, nvec = _as_rows(x, n, np.float64)
    y = np.empty_like(a)
    if _load().oracle_fwt_ld(_ptr(a, ctypes.c_double), _ptr(y, ctypes.c_double), nvec, n,
                             int(bool(normalize))) != 0:
        raise MemoryError("oracle_fwt_ld: allocation failed")
    return y.reshape(np.shape(x))


def fwt_kron(x, n, n1, normalize=False):
    """Kronecker-composed transform: n2 = n - n1 row bits, then n1 column
    bits, fp64."""
    a, nvec = _as_rows(x, n, np.float64)
    a = a.copy()
    rc = _load().oracle_fwt_kron_f64(_ptr(a, ctypes.c_double), nvec, n, n1,
                                     int(bool(normalize)))
    if rc != 0:
        raise ValueError("oracle_fwt_kron_f64 failed (n1=%d, n=%d)" % (n1, n))
    return a.reshape(np.shape(x))


def fwt_threaded_inplace(x, n, normalize, nthreads):
    """Timed-mode transform in place on a contiguous float32/float64 array
    with a pool of nthreads POSIX threads; returns the thread count used."""
    if not x.flags.c_contiguous:
        raise ValueError("x must be C-contiguous")
    N = 1 << n
    nvec = x.size // N
    lib = _load()
    if x.dtype == np.float32:
        return lib.oracle_fwt_threaded_f32(_ptr(x, ctypes.c_float), nvec, n,
                                           int(bool(normalize)), nthreads)
    if x.dtype == np.float64:
        return lib.oracle_fwt_threaded_f64(_ptr(x, ctypes.c_double), nvec, n,
                                           int(bool(normalize)), nthreads)
    raise TypeError("dtype must be float32 or float64")
