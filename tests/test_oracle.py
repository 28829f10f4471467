"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself: the hand-written
worked examples and Walsh matrix in tests/golden/ (from the entry
definition of the Apache Mahout pull request "[QDP] [feature] Pr4
kronecker fwt", section "How"), an independent numpy brute force,
scipy's Sylvester-construction Hadamard matrix, and textbook identities
(involution, Parseval, the Kronecker factorisation of the pull request's
"Why" section, the Sylvester recursion, the dyadic convolution theorem).
Each pin is also run against deliberately broken transforms (a dropped
stage, a flipped sign, a transposed index, a bit-reversed output, a wrong
normalisation) to show that a plausible mistake fails at least one pin.
"""
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
from oracle import brute_numpy
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(v) for v in line.split()])
    return np.array(rows)


def _ints(shape, seed):
    return np.random.default_rng(seed).integers(-8, 9, size=shape).astype(np.float64)


# ---- pins, each a function of a transform T(x, n, normalize) -> y ----------

def pin_golden_matrix(T):
    H = _read_rows("walsh_n3.txt")
    cols = np.stack([T(np.eye(8)[i], 3, False) for i in range(8)], axis=1)
    return np.array_equal(cols, H)


def pin_worked_example(T):
    x, y = _read_rows("worked_n3.txt")
    return np.array_equal(T(x, 3, False), y)


def pin_worked_complex(T):
    re, im, yre, yim = _read_rows("worked_n2_complex.txt")
    return np.array_equal(T(re, 2, True), yre) and np.array_equal(T(im, 2, True), yim)


def pin_numpy_bruteforce(T):
    for n in (1, 2, 3, 5, 7):
        x = _ints((3, 1 << n), 100 + n)
        if not np.array_equal(T(x, n, False), brute_numpy.bruteforce_int(x, n)):
            return False
    return True


def pin_scipy_hadamard(T):
    for n in (1, 4, 6):
        x = _ints((2, 1 << n), 200 + n)
        if not np.array_equal(T(x, n, False), x @ scipy.linalg.hadamard(1 << n).T):
            return False
    return True


def pin_involution(T):
    for n in (3, 6, 9):
        x = _ints((2, 1 << n), 300 + n)
        if not np.array_equal(T(T(x, n, False), n, False), x * (1 << n)):
            return False
    return True


def pin_parseval(T):
    for n in (4, 8):
        x = _ints((3, 1 << n), 400 + n)
        y = T(x, n, False).astype(np.int64)
        xi = x.astype(np.int64)
        if not np.array_equal((y * y).sum(axis=1), (xi * xi).sum(axis=1) << n):
            return False
    return True


def pin_sylvester_recursion(T):
    # H_n x = [H_{n-1}(a + b), H_{n-1}(a - b)] for x = [a, b].
    for n in (2, 5, 8):
        x = _ints(1 << n, 500 + n)
        a, b = x[: 1 << (n - 1)], x[1 << (n - 1):]
        want = np.concatenate([brute_numpy.bruteforce_int(a + b, n - 1),
                               brute_numpy.bruteforce_int(a - b, n - 1)])
        if not np.array_equal(T(x, n, False), want):
            return False
    return True


def pin_dyadic_convolution(T):
    # H(x * y) = (Hx)(Hy) for the dyadic (XOR) convolution.
    for n in (3, 6):
        N = 1 << n
        x, y = _ints(N, 600 + n), _ints(N, 700 + n)
        k = np.arange(N)
        conv = np.array([np.dot(x, y[np.bitwise_xor(kk, k)]) for kk in range(N)])
        if not np.array_equal(T(conv, n, False), T(x, n, False) * T(y, n, False)):
            return False
    return True


def pin_normalisation(T):
    for n in (2, 4, 6, 8):
        x = _ints(1 << n, 800 + n)
        if not np.array_equal(T(x, n, True), T(x, n, False) / 2.0 ** (n // 2)):
            return False
    return True


PINS = [pin_golden_matrix, pin_worked_example, pin_worked_complex, pin_numpy_bruteforce,
        pin_scipy_hadamard, pin_involution, pin_parseval, pin_sylvester_recursion,
        pin_dyadic_convolution, pin_normalisation]


def oracle_T(x, n, normalize):
    return oracle.fwt(x, n, normalize)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    assert pin(oracle_T)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_bruteforce_passes_pin(pin):
    """The C brute force from the definition satisfies the same pins."""
    assert pin(lambda x, n, nz: oracle.bruteforce(x, n, nz))


# ---- mutants: plausible mistakes, each must fail some pin ------------------

def _textbook(x, n, normalize, *, skip_stage=None, swap_sign_stage=None, scale=None):
    a = np.array(x, dtype=np.float64).reshape(-1, 1 << n).copy()
    N = 1 << n
    for s in range(n):
        if s == skip_stage:
            continue
        h = 1 << s
        for i in range(0, N, 2 * h):
            lo, hi = a[:, i:i + h].copy(), a[:, i + h:i + 2 * h].copy()
            if s == swap_sign_stage:
                a[:, i:i + h], a[:, i + h:i + 2 * h] = lo - hi, lo + hi
            else:
                a[:, i:i + h], a[:, i + h:i + 2 * h] = lo + hi, lo - hi
    if normalize:
        a *= scale if scale is not None else 2.0 ** (-n / 2)
    return a.reshape(np.shape(x))


def _bitrev(v, n):
    return int(format(v, "0%db" % n)[::-1], 2) if n else 0


MUTANTS = {
    "drop_last_stage": lambda x, n, nz: _textbook(x, n, nz, skip_stage=n - 1),
    "drop_first_stage": lambda x, n, nz: _textbook(x, n, nz, skip_stage=0),
    "sign_swapped_stage1": lambda x, n, nz: _textbook(x, n, nz, swap_sign_stage=1 if n > 1 else 0),
    "bit_reversed_output": lambda x, n, nz: _textbook(x, n, nz)[..., [_bitrev(k, n) for k in range(1 << n)]],
    "transposed_kron": lambda x, n, nz: _kron_transposed(x, n, nz),
    "normalise_by_2^-n": lambda x, n, nz: _textbook(x, n, nz, scale=2.0 ** (-n)),
    "sequency_order": lambda x, n, nz: _textbook(x, n, nz)[..., _sequency_perm(n)],
}


def _kron_transposed(x, n, normalize):
    # Row and column factors applied, but the result left in transposed
    # (column-major) order: the classic missing transpose-back.
    n1 = n // 2
    y = _textbook(x, n, normalize).reshape(-1, 1 << n1, 1 << (n - n1))
    return np.ascontiguousarray(np.swapaxes(y, 1, 2)).reshape(np.shape(x))


def _sequency_perm(n):
    N = 1 << n
    gray_inv = [k ^ (k >> 1) for k in range(N)]
    return [_bitrev(g, n) for g in gray_inv]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    failed = [p.__name__ for p in PINS if not p(MUTANTS[name])]
    assert failed, "mutant %s passes every pin" % name


def test_unmutated_reference_transform_passes_all_pins():
    """The same numpy textbook transform without a planted mistake passes."""
    for p in PINS:
        assert p(lambda x, n, nz: _textbook(x, n, nz)), p.__name__


# ---- direct checks -----------------------------------------------------------

@pytest.mark.parametrize("n", range(0, 11))
def test_textbook_equals_bruteforce_exactly(n):
    x = _ints((3, 1 << n), 900 + n)
    assert np.array_equal(oracle.fwt(x, n), oracle.bruteforce(x, n))
    assert np.array_equal(oracle.bruteforce(x, n), brute_numpy.bruteforce_int(x, n))


@pytest.mark.parametrize("n", [0, 1, 2, 5, 9, 12])
def test_closed_forms(n):
    N = 1 << n
    e0 = np.zeros(N)
    e0[0] = 1
    assert np.array_equal(oracle.fwt(e0, n), np.ones(N))
    ones = np.ones(N)
    want = np.zeros(N)
    want[0] = N
    assert np.array_equal(oracle.fwt(ones, n), want)


def test_n1_pair():
    assert np.array_equal(oracle.fwt(np.array([3.0, 5.0]), 1), [8.0, -2.0])


def test_n0_identity():
    x = np.array([[2.5], [-1.0]])
    assert np.array_equal(oracle.fwt(x, 0, True), x)
    assert np.array_equal(oracle.fwt(x, 0, False), x)


@pytest.mark.parametrize("n", [4, 7, 10, 13])
def test_kronecker_every_split_exact(n):
    x = _ints((2, 1 << n), 1000 + n)
    ref = oracle.fwt(x, n)
    for n1 in range(0, n + 1):
        assert np.array_equal(oracle.fwt_kron(x, n, n1), ref), n1


def test_kronecker_rejects_bad_split():
    with pytest.raises(ValueError):
        oracle.fwt_kron(np.zeros(8), 3, 4)


def test_linearity_exact():
    n = 9
    x, y = _ints(1 << n, 1), _ints(1 << n, 2)
    assert np.array_equal(oracle.fwt(3 * x - 2 * y, n), 3 * oracle.fwt(x, n) - 2 * oracle.fwt(y, n))


def test_rows_of_transform_are_orthogonal():
    n = 6
    N = 1 << n
    H = np.stack([oracle.fwt(np.eye(N)[i], n) for i in range(N)], axis=1)
    assert np.array_equal(H @ H.T, N * np.eye(N))
    assert np.array_equal(H, H.T)


@pytest.mark.parametrize("n", range(0, 16))
def test_norm_constant(n):
    c = float(oracle.norm_constant(n))
    assert c * c * (1 << n) == pytest.approx(1.0, rel=1e-15)
    if n % 2 == 0:
        assert c == 2.0 ** (-n // 2)
    c32 = oracle.norm_constant(n, np.float32)
    assert c32 == np.float32(c)


@pytest.mark.parametrize("n", [10, 16, 20])
def test_fp32_timed_mode_within_first_order_bound(n):
    # Each stage has norm sqrt(2) and adds at most u relative error per
    # output, so ||err||_2 <= n * u * 2^(n/2) * ||x||_2 to first order.
    rng = np.random.default_rng(n)
    x = rng.standard_normal((2, 1 << n)).astype(np.float32)
    y32 = oracle.fwt(x, n, False, dtype=np.float32).astype(np.float64)
    y64 = oracle.fwt(x.astype(np.float64), n, False)
    u = 2.0 ** -24
    for b in range(2):
        bound = n * u * 2 ** (n / 2) * np.linalg.norm(x[b].astype(np.float64))
        assert np.linalg.norm(y32[b] - y64[b]) <= 1.01 * bound


def test_fp64_normalised_parseval_gaussian():
    w = workloads.custom(12, 4, "f64", "gauss", True, seed=3)
    re, im = workloads.gen(w)
    yre, yim = oracle.fwt_complex(re, im, 12, normalize=True)
    for b in range(4):
        nx = np.sqrt(np.sum(re[b] ** 2) + np.sum(im[b] ** 2))
        ny = np.sqrt(np.sum(yre[b] ** 2) + np.sum(yim[b] ** 2))
        assert abs(ny - nx) <= 1e-13
        assert abs(nx - 1.0) <= 1e-14   # inputs are unit vectors


def test_threaded_matches_serial_and_reports_threads():
    n = 12
    x = np.random.default_rng(7).standard_normal((16, 1 << n)).astype(np.float32)
    y = x.copy()
    used = oracle.fwt_threaded_inplace(y, n, True, 4)
    assert used == 4
    assert np.array_equal(y, oracle.fwt(x, n, True, dtype=np.float32))
    z = x.astype(np.float64)
    assert oracle.fwt_threaded_inplace(z, n, False, 3) == 3
    assert np.array_equal(z, oracle.fwt(x.astype(np.float64), n, False))


@pytest.mark.parametrize("n", [0, 1, 3, 8, 10])
def test_long_double_transform_equals_bruteforce_on_integers(n):
    """The extended-precision network reaches the definition exactly on
    integer inputs (every partial sum is an integer far below 2^53)."""
    x = np.random.default_rng(500 + n).integers(-8, 9, size=(3, 1 << n)).astype(np.float64)
    assert np.array_equal(oracle.fwt_ld(x, n, False), oracle.bruteforce(x, n, False))
    if n % 2 == 0:
        assert np.array_equal(oracle.fwt_ld(x, n, True), oracle.bruteforce(x, n, True))


@pytest.mark.parametrize("n", [12, 13, 16, 17, 20])
def test_fp64_check_mode_against_long_double(n):
    """The fp64 check mode against the same network in long double: each of
    the n stages rounds once (relative error 2^-53 per output; every stage
    of the unnormalised network has norm sqrt(2), so the 2-norm of the
    accumulated error stays within n * 2^-53 * 2^(n/2) * ||x||), the scale
    rounds once more, and the long-double result is rounded to double once:
    max |fp64 - long double| <= (n + 2) * 2^-53 * ||x|| after
    normalisation.  That is at least 10^3 below the 1e-12 * ||x|| fp64
    tolerance of the GPU comparisons."""
    x = np.random.default_rng(600 + n).standard_normal((2, 1 << n))
    y64 = oracle.fwt(x, n, True)
    yld = oracle.fwt_ld(x, n, True)
    for b in range(2):
        nx = np.sqrt(np.sum(x[b] ** 2))
        err = np.abs(y64[b] - yld[b]).max()
        assert err <= (n + 2) * 2.0 ** -53 * nx, (b, err / nx)
        assert err <= 1e-15 * nx
    # and the long-double result keeps the norm to far better than fp64
    nld = np.sqrt(np.sum(yld.astype(np.longdouble) ** 2, axis=1))
    assert np.abs(nld - np.sqrt(np.sum(x.astype(np.longdouble) ** 2, axis=1))).max() <= 1e-14
