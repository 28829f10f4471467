"""Property-based pins of the CPU oracle (no GPU), with Hypothesis over
n <= 10 and integer inputs in [-8, 8], where every sum is an exact integer
and every identity below holds exactly:

* agreement with the numpy brute force of the entry definition
  y_k = sum_i (-1)^popcount(k AND i) x_i (the Apache Mahout pull request
  "[QDP] [feature] Pr4 kronecker fwt", section "How");
* involution H H = 2^n I, and Parseval ||Hx||^2 = 2^n ||x||^2 (in int64);
* linearity;
* the Kronecker split H_n = H_{n1} (x) H_{n - n1} for any n1 (the pull
  request's "Why" section);
* invariance under a common permutation of the index bits of input and
  output (popcount(k AND i) does not change);
* the dyadic convolution theorem H(x * y) = Hx . Hy with
  (x * y)_k = sum_i x_i y_(k XOR i), divided by 2^n on the left.
"""
import numpy as np
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

import oracle  # noqa: E402
from oracle import brute_numpy  # noqa: E402

SETTINGS = settings(max_examples=60, deadline=None, derandomize=True)


@st.composite
def int_vectors(draw, nmax=10, batch_max=3):
    n = draw(st.integers(0, nmax))
    b = draw(st.integers(1, batch_max))
    seed = draw(st.integers(0, 2**32 - 1))
    x = np.random.default_rng(seed).integers(-8, 9, size=(b, 1 << n)).astype(np.float64)
    return n, x


@SETTINGS
@given(int_vectors())
def test_matches_bruteforce(nx):
    n, x = nx
    assert np.array_equal(oracle.fwt(x.copy(), n), brute_numpy.bruteforce(x, n))


@SETTINGS
@given(int_vectors())
def test_involution_and_parseval(nx):
    n, x = nx
    y = oracle.fwt(x.copy(), n)
    assert np.array_equal(oracle.fwt(y.copy(), n), x * 2.0 ** n)
    xi, yi = x.astype(np.int64), y.astype(np.int64)
    assert np.array_equal((yi * yi).sum(axis=-1), (xi * xi).sum(axis=-1) << n)


@SETTINGS
@given(int_vectors(), st.integers(-3, 3), st.integers(-3, 3), st.integers(0, 2**32 - 1))
def test_linearity(nx, a, b, seed):
    n, x = nx
    y = np.random.default_rng(seed).integers(-8, 9, size=x.shape).astype(np.float64)
    lhs = oracle.fwt(a * x + b * y, n)
    assert np.array_equal(lhs, a * oracle.fwt(x.copy(), n) + b * oracle.fwt(y.copy(), n))


@SETTINGS
@given(int_vectors(), st.data())
def test_kronecker_split(nx, data):
    n, x = nx
    n1 = data.draw(st.integers(0, n))
    assert np.array_equal(oracle.fwt_kron(x.copy(), n, n1), oracle.fwt(x.copy(), n))


@SETTINGS
@given(int_vectors(nmax=8), st.randoms(use_true_random=False))
def test_index_bit_permutation(nx, rnd):
    n, x = nx
    perm = list(range(n))
    rnd.shuffle(perm)
    idx = np.arange(1 << n)
    moved = np.zeros_like(idx)
    for b, to in enumerate(perm):
        moved |= ((idx >> b) & 1) << to
    px = np.empty_like(x)
    px[:, moved] = x          # (P x)_{pi(i)} = x_i
    hy = oracle.fwt(x.copy(), n)
    phy = np.empty_like(hy)
    phy[:, moved] = hy
    assert np.array_equal(oracle.fwt(px, n), phy)


@SETTINGS
@given(int_vectors(nmax=7, batch_max=1), st.integers(0, 2**32 - 1))
def test_dyadic_convolution(nx, seed):
    n, x = nx
    x = x[0]
    y = np.random.default_rng(seed).integers(-8, 9, size=x.shape).astype(np.float64)
    N = 1 << n
    k = np.arange(N)
    conv = np.array([np.dot(x, y[k ^ j]) for j in range(N)])
    assert np.array_equal(oracle.fwt(conv.copy(), n),
                          oracle.fwt(x.copy(), n) * oracle.fwt(y.copy(), n))
