"""Second, independent brute-force oracle written with numpy.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Builds the Walsh matrix from its entry definition, (-1)^popcount(k & i)
(Apache Mahout pull request "[QDP] [feature] Pr4 kronecker fwt", section
"How"), with numpy's bitwise_count, and multiplies.  It shares nothing
with oracle.c, so agreement between the two pins the sign convention and
the natural output order.
"""
import numpy as np


def walsh_matrix(n):
    """Dense 2^n x 2^n matrix with entries (-1)^popcount(k & i), int64."""
    idx = np.arange(1 << n, dtype=np.uint64)
    parity = np.bitwise_count(np.bitwise_and.outer(idx, idx)) & 1
    return (1 - 2 * parity.astype(np.int64))


def bruteforce(x, n, normalize=False):
    """y = c * W x for every length-2^n row of x (float64)."""
    a = np.asarray(x, dtype=np.float64).reshape(-1, 1 << n)
    y = a @ walsh_matrix(n).T.astype(np.float64)
    if normalize:
        y = y / np.sqrt(np.float64(1 << n))
    return y.reshape(np.shape(x))


def bruteforce_int(x, n):
    """Exact integer transform of integer rows (int64 arithmetic)."""
    a = np.asarray(x, dtype=np.int64).reshape(-1, 1 << n)
    return (a @ walsh_matrix(n).T).reshape(np.shape(x))
