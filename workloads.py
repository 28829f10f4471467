"""Seeded synthetic workloads for the batched Walsh-Hadamard transform.

This module holds the workload table and the input generators that both
the HIP path's tests/benchmark and the oracle consume.  It holds none of
the transform's arithmetic.

Generator recipe (every vector independent, so any single vector can be
regenerated on its own for sampled checks of the full-size workloads):

* vector b of a workload with seed s draws from
  ``numpy.random.default_rng([s, b])`` (PCG64 seeded through SeedSequence),
  first the N = 2^n real parts, then the N imaginary parts;
* "int" workloads draw integers uniform on {-8, ..., 8} (inclusive);
* "gauss" workloads draw standard normals in float64, divide both parts by
  the vector's complex 2-norm sqrt(sum re^2 + sum im^2) (float64), then
  cast once to the workload's dtype.

The pages measure on no public dataset; these synthetic states stand in
for the IQP-encoder inputs of the Apache Mahout pull request
"[QDP] [feature] Pr4 kronecker fwt" (section "Benchmark Results": batch 64
at 12 and 14 qubits), extended to the 20- and 24-qubit sizes.
"""
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
import os

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    n: int              # qubits; each vector has 2^n complex amplitudes
    batch: int          # complex vectors
    dtype: str          # "f32" or "f64"
    values: str         # "int" or "gauss"
    normalize: bool     # multiply by 2^(-n/2)
    seed: int
    split: tuple = ()   # explicit Kronecker split (row bits first), or () for auto

    @property
    def N(self):
        return 1 << self.n

    @property
    def np_dtype(self):
        return np.float32 if self.dtype == "f32" else np.float64

    @property
    def itemsize(self):
        return 4 if self.dtype == "f32" else 8

    @property
    def state_bytes(self):
        """S: bytes of the planar state (re + im)."""
        return 2 * self.batch * self.N * self.itemsize


WORKLOADS = {
    "n10_b8_f32_int": Workload("n10_b8_f32_int", 10, 8, "f32", "int", False, 10),
    "n12_b64_f32": Workload("n12_b64_f32", 12, 64, "f32", "gauss", True, 12),
    "n14_b64_f32": Workload("n14_b64_f32", 14, 64, "f32", "gauss", True, 14, (7, 7)),
    "n20_b256_f32": Workload("n20_b256_f32", 20, 256, "f32", "gauss", True, 20),
    "n24_b16_f64": Workload("n24_b16_f64", 24, 16, "f64", "gauss", True, 24),
}


def gen_vector(w, b):
    """(re, im) of vector b of workload w, as arrays of w's dtype."""
    rng = np.random.default_rng([w.seed, b])
    if w.values == "int":
        re = rng.integers(-8, 9, size=w.N)
        im = rng.integers(-8, 9, size=w.N)
        return re.astype(w.np_dtype), im.astype(w.np_dtype)
    re = rng.standard_normal(w.N)
    im = rng.standard_normal(w.N)
    nrm = np.sqrt(np.dot(re, re) + np.dot(im, im))
    return (re / nrm).astype(w.np_dtype), (im / nrm).astype(w.np_dtype)


def gen(w, out_re=None, out_im=None, threads=None):
    """Whole batch (re, im), each of shape (batch, N).

    ``out_re``/``out_im`` may be preallocated (e.g. pinned) arrays of the
    right shape and dtype; vectors are generated in parallel threads.
    """
    shape = (w.batch, w.N)
    re = np.empty(shape, w.np_dtype) if out_re is None else out_re
    im = np.empty(shape, w.np_dtype) if out_im is None else out_im
    if re.shape != shape or im.shape != shape:
        raise ValueError("output arrays must have shape %s" % (shape,))

    def one(b):
        re[b], im[b] = gen_vector(w, b)

    threads = threads or min(16, len(os.sched_getaffinity(0)))
    if w.batch * w.N <= (1 << 16) or threads <= 1:
        for b in range(w.batch):
            one(b)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(w.batch)))
    return re, im


def custom(n, batch, dtype="f32", values="gauss", normalize=True, seed=0):
    """An ad-hoc workload with the same recipe (used by sweeps and edge cases)."""
    return Workload("custom_n%d_b%d_%s_%s" % (n, batch, dtype, values), n, batch,
                    dtype, values, normalize, seed)
