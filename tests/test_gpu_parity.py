"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars:
* integer inputs (U{-8..8}) unnormalised, and normalised at even n:
  bit-exact (every partial sum is an integer below 2^24, so every order of
  evaluation is exact, and 2^(-n/2) is a power of two);
* Gaussian unit-norm inputs, normalised: max |err| <= 1e-5 * ||x||_2
  (fp32) or 1e-12 * ||x||_2 (fp64) per vector, ||x||_2 the complex 2-norm
  of the input after the cast, the error measured against the fp64
  oracle.
The full-size workloads are checked on sampled vectors that the oracle
transforms one by one, plus norm preservation (Parseval) of every vector.
"""
import ctypes
import sys

import numpy as np
import pytest

import oracle
import quantum_state_encoding_amd as qse
import workloads
from plan_cases import (FORCED_SPLITS, LDS_SINGLE_CASES, LX_CASES, LX_COLUMN_CASES, LX_PHASE_CASES,
                        PIPE_CASES, VARIANTS, WAVE_CASES, random_plan_cases)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

TOL = {"f32": 1e-5, "f64": 1e-12}


def say(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def run(plan, re, im, normalize, stream=None):
    tre, tim = to_dev(re), (to_dev(im) if im is not None else None)
    plan.execute(tre, tim, normalize=normalize, stream=stream)
    torch.cuda.synchronize()
    return tre.cpu().numpy(), (tim.cpu().numpy() if tim is not None else None)


def ints(shape, seed, dtype):
    return np.random.default_rng(seed).integers(-8, 9, size=shape).astype(dtype)


def assert_exact(got, re, n, normalize):
    want = oracle.fwt(re, n, normalize)
    assert np.array_equal(got.astype(np.float64), want)


def assert_close(w_dtype, n, re, im, gre, gim, normalize=True):
    ore, oim = oracle.fwt_complex(re, im, n, normalize)
    re2, im2 = re.reshape(-1, 1 << n), im.reshape(-1, 1 << n)
    for b in range(re2.shape[0]):
        nx = np.sqrt(np.sum(re2[b].astype(np.float64) ** 2) + np.sum(im2[b].astype(np.float64) ** 2))
        bound = TOL[w_dtype] * nx * (1.0 if normalize else 2.0 ** (n / 2))
        err = max(np.abs(gre.reshape(re2.shape)[b] - ore.reshape(re2.shape)[b]).max(),
                  np.abs(gim.reshape(re2.shape)[b] - oim.reshape(re2.shape)[b]).max())
        assert err <= bound, "vector %d: max|err| %.3g > %.3g" % (b, err, bound)


# ---- the small workloads, as configured ------------------------------------

def test_n10_b8_integer_bit_exact():
    w = workloads.WORKLOADS["n10_b8_f32_int"]
    say(w.name)
    re, im = workloads.gen(w)
    gre, gim = run(qse.Plan(w.n, w.dtype), re, im, w.normalize)
    assert_exact(gre, re, w.n, False)
    assert_exact(gim, im, w.n, False)


@pytest.mark.parametrize("name,split", [("n12_b64_f32", None), ("n14_b64_f32", (7, 7)),
                                        ("n14_b64_f32", None)])
def test_gaussian_workloads(name, split):
    w = workloads.WORKLOADS[name]
    say("%s split=%s" % (name, split))
    re, im = workloads.gen(w)
    plan = qse.Plan(w.n, w.dtype, split=split)
    gre, gim = run(plan, re, im, True)
    assert_close(w.dtype, w.n, re, im, gre, gim)


# ---- exact sweeps over n, dtype and batch ------------------------------------

@pytest.mark.parametrize("dtype,n", [("f32", n) for n in range(0, 21)] +
                         [("f64", n) for n in range(0, 25)])
def test_integer_sweep_auto_plan(dtype, n):
    say("sweep %s n=%d" % (dtype, n))
    batch = 3 if n <= 18 else 1
    npd = np.float32 if dtype == "f32" else np.float64
    re = ints((batch, 1 << n), 10_000 + n, npd)
    im = ints((batch, 1 << n), 20_000 + n, npd)
    plan = qse.Plan(n, dtype)
    gre, gim = run(plan, re, im, False)
    assert_exact(gre, re, n, False)
    assert_exact(gim, im, n, False)
    if n % 2 == 0:   # normalised by an exact power of two
        gre, gim = run(plan, re, im, True)
        assert_exact(gre, re, n, True)
        assert_exact(gim, im, n, True)


@pytest.mark.parametrize("dtype,n", LDS_SINGLE_CASES)
def test_integer_lds_tile_single_pass(dtype, n):
    """The LDS-tile kernel on the small one-pass sizes whose default plan
    takes the wave-tile kernel, exactly, unnormalised and normalised."""
    say("lds tile %s n=%d" % (dtype, n))
    npd = np.float32 if dtype == "f32" else np.float64
    re = ints((5, 1 << n), 12_000 + n, npd)
    im = ints((5, 1 << n), 22_000 + n, npd)
    plan = qse.Plan(n, dtype, split=(n,), wave=(0,))
    for normalize in (False, True):
        if normalize and n % 2:
            continue
        gre, gim = run(plan, re, im, normalize)
        assert_exact(gre, re, n, normalize)
        assert_exact(gim, im, n, normalize)


@pytest.mark.parametrize("dtype,n,split", FORCED_SPLITS)
def test_integer_forced_splits(dtype, n, split):
    say("split %s n=%d %s" % (dtype, n, split))
    npd = np.float32 if dtype == "f32" else np.float64
    re = ints((2, 1 << n), 30_000 + n, npd)
    im = ints((2, 1 << n), 40_000 + n, npd)
    plan = qse.Plan(n, dtype, split=split)
    assert plan.pass_bits == list(split)
    gre, gim = run(plan, re, im, False)
    assert_exact(gre, re, n, False)
    assert_exact(gim, im, n, False)


@pytest.mark.parametrize("dtype,n,split,eb,gbits,phases", VARIANTS)
def test_integer_kernel_variants(dtype, n, split, eb, gbits, phases):
    say("variant %s n=%d split=%s eb=%s gbits=%s phases=%s" % (dtype, n, split, eb, gbits, phases))
    npd = np.float32 if dtype == "f32" else np.float64
    re = ints((2, 1 << n), 50_000 + n, npd)
    im = ints((2, 1 << n), 60_000 + n, npd)
    plan = qse.Plan(n, dtype, split=split, eb=eb, gbits=gbits, phases=phases)
    gre, gim = run(plan, re, im, False)
    assert_exact(gre, re, n, False)
    assert_exact(gim, im, n, False)


@pytest.mark.parametrize("dtype,n,split,eb,pipe,batch", PIPE_CASES)
def test_integer_pipelined_kernels(dtype, n, split, eb, pipe, batch):
    """The persistent software-pipelined kernel (each workgroup walks several
    tile groups and prefetches the next) against the oracle, exactly."""
    say("pipe %s n=%d split=%s eb=%s pipe=%s batch=%d" % (dtype, n, split, eb, pipe, batch))
    npd = np.float32 if dtype == "f32" else np.float64
    plan = qse.Plan(n, dtype, split=split, eb=eb, pipe=pipe)
    for i, pv in enumerate(pipe):
        if pv >= 0:
            assert plan.pass_config(i)["pipe"] == pv
    re = ints((batch, 1 << n), 95_000 + n, npd)
    im = ints((batch, 1 << n), 96_000 + n, npd)
    gre, gim = run(plan, re, im, False)
    assert_exact(gre, re, n, False)
    assert_exact(gim, im, n, False)


@pytest.mark.parametrize("dtype,n,split,eb,gbits,wave,batch", WAVE_CASES)
def test_integer_wave_tile_kernels(dtype, n, split, eb, gbits, wave, batch):
    """The wave-tile kernel: register butterflies plus lane stages (DPP quad
    permutes, ds_swizzle, permlane16/32 swaps), exactly against the oracle,
    unnormalised and normalised."""
    say("wave %s n=%d split=%s eb=%s gbits=%s wave=%s batch=%d" % (dtype, n, split, eb, gbits,
                                                                     wave, batch))
    npd = np.float32 if dtype == "f32" else np.float64
    plan = qse.Plan(n, dtype, split=split, eb=eb, gbits=gbits, wave=wave)
    for i, wv in enumerate(wave):
        assert plan.pass_config(i)["wave"] == wv
    re = ints((batch, 1 << n), 97_000 + n, npd)
    im = ints((batch, 1 << n), 98_000 + n, npd)
    gre, gim = run(plan, re, im, False)
    assert_exact(gre, re, n, False)
    assert_exact(gim, im, n, False)
    if n % 2 == 0:
        gre, gim = run(plan, re, im, True)
        assert_exact(gre, re, n, True)
        assert_exact(gim, im, n, True)


@pytest.mark.parametrize("dtype,n,split,eb,wave,batch", LX_CASES)
def test_integer_lane_exchange_kernels(dtype, n, split, eb, wave, batch):
    """The lane-exchange row kernel: register and lane stages, one LDS
    exchange of the wave bits, exactly against the oracle, unnormalised and
    normalised."""
    say("lx %s n=%d split=%s eb=%s wave=%s batch=%d" % (dtype, n, split, eb, wave, batch))
    npd = np.float32 if dtype == "f32" else np.float64
    plan = qse.Plan(n, dtype, split=split, eb=eb, wave=wave)
    for i, wv in enumerate(wave):
        assert plan.pass_config(i)["wave"] == wv
    re = ints((batch, 1 << n), 99_000 + n, npd)
    im = ints((batch, 1 << n), 99_500 + n, npd)
    gre, gim = run(plan, re, im, False)
    assert_exact(gre, re, n, False)
    assert_exact(gim, im, n, False)
    if n % 2 == 0:
        gre, gim = run(plan, re, im, True)
        assert_exact(gre, re, n, True)
        assert_exact(gim, im, n, True)


@pytest.mark.parametrize("dtype,n,split,eb,wave,batch",
                         [c for c in LX_CASES if c[1] % 2 == 1])
def test_gaussian_lane_exchange_kernels_odd_n(dtype, n, split, eb, wave, batch):
    """The lane-exchange kernels at odd n, normalised: the scale is not a
    power of two there, and fp32 row tiles fuse it with their last
    butterfly (a different rounding from a separate multiply), so these
    are compared within the tolerance, on Gaussian states."""
    say("lx gauss %s n=%d split=%s eb=%s wave=%s batch=%d" % (dtype, n, split, eb, wave, batch))
    plan = qse.Plan(n, dtype, split=split, eb=eb, wave=wave)
    w = workloads.custom(n, batch, dtype, "gauss", True, seed=91_000 + n)
    re, im = workloads.gen(w)
    gre, gim = run(plan, re, im, True)
    assert_close(dtype, n, re, im, gre, gim)


# (dtype, n, split, batch, wave): multi-pass plans on states below 256 MiB
# with at least 8 vectors, whose launches place each vector component's
# workgroups on one XCD (all of them, or the first multiple of 8), in each
# kernel family
XCD_CASES = [("f32", 14, (7, 7), 64, None), ("f32", 14, (7, 7), 8, (1, 1)),
             ("f32", 14, (7, 7), 16, (0, 0)), ("f32", 12, (6, 6), 64, None),
             ("f32", 16, (9, 7), 16, None), ("f32", 18, (11, 7), 8, None),
             ("f32", 15, (5, 5, 5), 64, None), ("f32", 16, (10, 6), 24, None),
             ("f64", 14, (7, 7), 32, None), ("f64", 16, (8, 8), 8, None),
             ("f64", 13, (7, 6), 64, (1, 1)), ("f32", 16, (10, 6), 13, None),
             ("f32", 20, (12, 8), 12, None)]


@pytest.mark.parametrize("dtype,n,split,batch,wave", XCD_CASES)
def test_integer_xcd_placed_passes(dtype, n, split, batch, wave):
    """Small multi-pass states, where each pass runs every vector
    component's workgroups on one XCD (a permutation of the launch's
    workgroups): exact against the oracle, unnormalised and normalised."""
    say("xcd %s n=%d split=%s batch=%d wave=%s" % (dtype, n, split, batch, wave))
    npd = np.float32 if dtype == "f32" else np.float64
    plan = qse.Plan(n, dtype, split=split, wave=wave) if wave else qse.Plan(n, dtype, split=split)
    re = ints((batch, 1 << n), 93_000 + n, npd)
    im = ints((batch, 1 << n), 94_000 + n, npd)
    for normalize in ((False, True) if n % 2 == 0 else (False,)):
        gre, gim = run(plan, re, im, normalize)
        assert_exact(gre, re, n, normalize)
        assert_exact(gim, im, n, normalize)


@pytest.mark.parametrize("dtype,n,split,eb,batch", LX_PHASE_CASES)
def test_integer_lane_exchange_phases(dtype, n, split, eb, batch):
    """The lane-exchange kernel with its exchange in two phases through
    half the LDS, exactly against the oracle."""
    say("lx phases %s n=%d split=%s eb=%s batch=%d" % (dtype, n, split, eb, batch))
    npd = np.float32 if dtype == "f32" else np.float64
    rest = (-1,) * (len(split) - 1)
    plan = qse.Plan(n, dtype, split=split, eb=eb, phases=(1,) + rest, wave=(2,) + rest)
    assert plan.pass_config(0)["phase_bits"] == 1
    re = ints((batch, 1 << n), 99_700 + n, npd)
    im = ints((batch, 1 << n), 99_800 + n, npd)
    gre, gim = run(plan, re, im, False)
    assert_exact(gre, re, n, False)
    assert_exact(gim, im, n, False)
    if n % 2 == 0:
        gre, gim = run(plan, re, im, True)
        assert_exact(gre, re, n, True)
        assert_exact(gim, im, n, True)


def lx_column_plan(dtype, n, split, eb, gbits, phases):
    k = len(split)
    knobs = {name: tuple(v if i == 1 else -1 for i in range(k))
             for name, v in (("eb", eb), ("gbits", gbits), ("phases", phases), ("wave", 2))}
    return qse.Plan(n, dtype, split=split, **knobs)


@pytest.mark.parametrize("dtype,n,split,eb,gbits,phases,batch", LX_COLUMN_CASES)
def test_integer_lane_exchange_columns(dtype, n, split, eb, gbits, phases, batch):
    """The lane-exchange kernel on a column pass (lanes hold the column
    groups and the lowest row bits), exactly against the oracle."""
    say("lx column %s n=%d split=%s eb=%d gbits=%d phases=%d batch=%d" % (
        dtype, n, split, eb, gbits, phases, batch))
    npd = np.float32 if dtype == "f32" else np.float64
    plan = lx_column_plan(dtype, n, split, eb, gbits, phases)
    assert plan.pass_config(1)["wave"] == 2
    re = ints((batch, 1 << n), 99_900 + n, npd)
    im = ints((batch, 1 << n), 99_950 + n, npd)
    gre, gim = run(plan, re, im, False)
    assert_exact(gre, re, n, False)
    assert_exact(gim, im, n, False)
    if n % 2 == 0:
        gre, gim = run(plan, re, im, True)
        assert_exact(gre, re, n, True)
        assert_exact(gim, im, n, True)


def _planner_accepts(dtype, n, split, kw):
    try:
        qse.Plan(n, dtype, split=split, **kw)
        return True
    except qse.FwtError:
        return False


RANDOM_CASES = random_plan_cases(_planner_accepts)
# the same with 8-24 vectors, so that multi-pass launches place their
# workgroups by XCD (all of them, or the first multiple of 8)
RANDOM_XCD_CASES = random_plan_cases(_planner_accepts, count=40, seed=20_261_203,
                                     batches=(8, 11, 16, 24))


@pytest.mark.parametrize("dtype,n,split,kw,batch,modes", RANDOM_CASES + RANDOM_XCD_CASES,
                         ids=["r%02d-%s-n%d-%s" % (i, c[0], c[1], "-".join(c[5]))
                              for i, c in enumerate(RANDOM_CASES)] +
                             ["x%02d-%s-n%d-b%d-%s" % (i, c[0], c[1], c[4], "-".join(c[5]))
                              for i, c in enumerate(RANDOM_XCD_CASES)])
def test_integer_random_plans(dtype, n, split, kw, batch, modes):
    """Seeded random plans (1-4 factors, each pass on its default kernel
    or with a kernel family and random tiling fields forced), exactly
    against the oracle."""
    say("random plan %s n=%d split=%s %s batch=%d" % (dtype, n, split, kw, batch))
    npd = np.float32 if dtype == "f32" else np.float64
    plan = qse.Plan(n, dtype, split=split, **kw)
    assert plan.pass_bits == list(split)
    seed = 123_000 + 31 * n + len(split)
    re = ints((batch, 1 << n), seed, npd)
    im = ints((batch, 1 << n), seed + 1, npd)
    for normalize in ((False, True) if n % 2 == 0 else (False,)):
        gre, gim = run(plan, re, im, normalize)
        assert_exact(gre, re, n, normalize)
        assert_exact(gim, im, n, normalize)


@pytest.mark.parametrize("dtype,n,batch", [("f32", 12, 1), ("f32", 12, 3), ("f32", 12, 257),
                                           ("f32", 8, 1001), ("f32", 16, 5), ("f64", 16, 3),
                                           ("f64", 6, 77), ("f32", 3, 9), ("f32", 1, 7),
                                           ("f64", 1, 5), ("f32", 2, 33)])
def test_ragged_batches(dtype, n, batch):
    say("batch %s n=%d batch=%d" % (dtype, n, batch))
    npd = np.float32 if dtype == "f32" else np.float64
    re = ints((batch, 1 << n), 70_000 + batch, npd)
    im = ints((batch, 1 << n), 80_000 + batch, npd)
    gre, gim = run(qse.Plan(n, dtype), re, im, False)
    assert_exact(gre, re, n, False)
    assert_exact(gim, im, n, False)


@pytest.mark.parametrize("dtype,n,batch", [("f32", 20, 37), ("f32", 21, 20), ("f64", 22, 5),
                                           ("f32", 20, 33)])
def test_integer_chunked_schedule(dtype, n, batch):
    """Calls larger than the Infinity Cache run in chunks of vectors
    (including a ragged last chunk); every vector must still be exact."""
    say("chunked %s n=%d batch=%d" % (dtype, n, batch))
    npd = np.float32 if dtype == "f32" else np.float64
    plan = qse.Plan(n, dtype)
    cv = plan.chunk_vectors(batch, True)
    assert 0 < cv < batch
    re = ints((batch, 1 << n), 85_000 + n, npd)
    im = ints((batch, 1 << n), 86_000 + n, npd)
    gre, gim = run(plan, re, im, False)
    for b in range(batch):
        assert_exact(gre[b], re[b], n, False)
        assert_exact(gim[b], im[b], n, False)


# Multi-pass calls whose stores leave the plain form: passes before the last
# store with device scope on states past the L2s (32 MiB) when their tiles
# have at most 2^10 16-byte slots, and the last pass stores nontemporally on
# states past the Infinity Cache (256 MiB).  The cases put every kernel
# family in such a pass.
STORE_CASES = [
    ("f32", 18, (9, 9), 40, dict(wave=(0, 0))),       # LDS-tile row: device scope
    ("f32", 18, (7, 11), 40, dict(wave=(1, 0))),      # wave-tile row: device scope
    ("f32", 20, (10, 10), 40, dict(wave=(1, 0))),     # LDS-tile column: nontemporal
    ("f32", 20, (12, 8), 40, dict(wave=(0, 1))),      # wave-tile column: nontemporal
    ("f64", 18, (9, 9), 72, dict(wave=(0, 0))),       # both, fp64
    ("f64", 20, (11, 9), 40, {}),                     # lane-exchange row and column
    ("f64", 20, (8, 12), 20, dict(pipe=(0, 1), wave=(0, 0))),   # pipelined column
    ("f32", 24, (8, 8, 8), 5, {}),                    # three passes on block chunks
]


@pytest.mark.parametrize("dtype,n,split,batch,kw", STORE_CASES)
def test_integer_store_policies(dtype, n, split, batch, kw):
    """Device-scope and nontemporal stores in every kernel family: each
    vector exact against the oracle."""
    say("stores %s n=%d split=%s batch=%d %s" % (dtype, n, split, batch, kw))
    npd = np.float32 if dtype == "f32" else np.float64
    plan = qse.Plan(n, dtype, split=split, **kw)
    # fp32 results stay exact integers while |x| 2^n <= 2^24
    lim = min(8, 1 << max(0, 24 - n)) if dtype == "f32" else 8
    re = np.random.default_rng(87_000 + n).integers(-lim, lim + 1, (batch, 1 << n)).astype(npd)
    im = np.random.default_rng(88_000 + n).integers(-lim, lim + 1, (batch, 1 << n)).astype(npd)
    gre, gim = run(plan, re, im, False)
    for b in range(batch):
        assert_exact(gre[b], re[b], n, False)
        assert_exact(gim[b], im[b], n, False)


# ---- floating point, odd n and the normalisation -----------------------------

@pytest.mark.parametrize("dtype,n", [("f32", n) for n in (3, 5, 11, 13, 15, 17, 19, 21, 23)] +
                         [("f64", n) for n in (3, 7, 13, 15, 19, 23)])
def test_gaussian_normalised_odd_and_large_n(dtype, n):
    say("gauss %s n=%d" % (dtype, n))
    w = workloads.custom(n, 2, dtype, "gauss", True, seed=90_000 + n)
    re, im = workloads.gen(w)
    gre, gim = run(qse.Plan(n, dtype), re, im, True)
    assert_close(dtype, n, re, im, gre, gim)


def test_unnormalised_gaussian_f32():
    n = 16
    say("gauss unnormalised n=16")
    w = workloads.custom(n, 3, "f32", "gauss", False, seed=5)
    re, im = workloads.gen(w)
    gre, gim = run(qse.Plan(n, "f32"), re, im, False)
    assert_close("f32", n, re, im, gre, gim, normalize=False)


# ---- the full-size workloads, in the benchmark's launch configuration --------

def _full_size(name, samples):
    """The workload the benchmark times, at its full size, in the plan it
    times: every vector compared element by element with the oracle's fp64
    transform (its threaded form, over blocks of vectors), plus norm
    preservation of every vector."""
    import os
    w = workloads.WORKLOADS[name]
    say("full size %s" % name)
    re, im = workloads.gen(w)
    plan = qse.Plan(w.n, w.dtype)          # the plan the benchmark times
    tre, tim = to_dev(re), to_dev(im)
    plan.execute(tre, tim, normalize=True)
    torch.cuda.synchronize()
    # Parseval for every vector: the normalised transform keeps the norm.
    ny = torch.sqrt((tre.double() ** 2).sum(1) + (tim.double() ** 2).sum(1)).cpu().numpy()
    nx = np.sqrt((re.astype(np.float64) ** 2).sum(1) + (im.astype(np.float64) ** 2).sum(1))
    assert np.abs(ny - nx).max() <= TOL[w.dtype] * nx.max()
    threads = min(16, len(os.sched_getaffinity(0)))
    blk = max(1, (64 << 20) // (w.N * 8))  # vectors per block: 64 MiB of fp64 per component
    worst = 0.0
    for b0 in range(0, w.batch, blk):
        b1 = min(w.batch, b0 + blk)
        o = np.concatenate([re[b0:b1], im[b0:b1]]).astype(np.float64)
        oracle.fwt_threaded_inplace(o, w.n, True, threads)
        g_re = tre[b0:b1].cpu().numpy().astype(np.float64)
        g_im = tim[b0:b1].cpu().numpy().astype(np.float64)
        err = np.maximum(np.abs(g_re - o[:b1 - b0]).max(1), np.abs(g_im - o[b1 - b0:]).max(1))
        ratio = err / nx[b0:b1]
        worst = max(worst, float(ratio.max()))
        assert (ratio <= TOL[w.dtype]).all(), "vectors %d..%d: max|err|/||x|| %.3g" % (
            b0, b1 - 1, ratio.max())
    say("full size %s: %d vectors, max|err|/||x|| = %.3g" % (name, w.batch, worst))
    for b in samples:
        # a sampled input regenerates on its own from the recipe
        r2, i2 = workloads.gen_vector(w, b)
        assert np.array_equal(r2, re[b]) and np.array_equal(i2, im[b])
    del tre, tim
    torch.cuda.empty_cache()


def test_full_size_n20_b256_f32():
    _full_size("n20_b256_f32", samples=(0, 1, 137, 255))


def test_full_size_n24_b16_f64():
    _full_size("n24_b16_f64", samples=(0, 9, 15))


@pytest.mark.parametrize("dtype,n,passes", [("f32", 24, 2), ("f32", 25, 2), ("f32", 26, 2),
                                            ("f32", 27, 3), ("f64", 25, 2), ("f64", 26, 3)])
def test_wide_default_plans(dtype, n, passes):
    """The default plans above n = 23 at their real size (two passes with
    10- and 11-bit column factors, then three, whose first two passes run
    on chunks of sub-vector blocks), one vector, inputs in {-1, 0, 1}: the
    partial sums stay exact integers far below 2^24, so the result is
    exact; compared whole with the oracle."""
    say("wide default plan %s n=%d" % (dtype, n))
    npd = np.float32 if dtype == "f32" else np.float64
    rng = np.random.default_rng(77_000 + n)
    re = rng.integers(-1, 2, size=(1, 1 << n)).astype(npd)
    im = rng.integers(-1, 2, size=(1, 1 << n)).astype(npd)
    plan = qse.Plan(n, dtype)
    assert plan.num_passes == passes
    if passes == 3:
        assert plan.call_schedule(1)[:2] == (2, sum(plan.pass_bits[:2]))
    gre, gim = run(plan, re, im, False)
    assert_exact(gre, re, n, False)
    assert_exact(gim, im, n, False)


@pytest.mark.parametrize("dtype,n,batch,split", [("f32", 27, 2, None), ("f64", 26, 1, None),
                                                 ("f32", 28, 1, (7, 7, 7, 7)),
                                                 ("f32", 27, 3, (10, 10, 7))])
def test_block_chunked_schedule_equals_passes_in_order(dtype, n, batch, split):
    """Vectors larger than the Infinity Cache: fwt_execute runs the leading
    passes on chunks of sub-vector blocks (fwt_plan_call_schedule), which
    must give bit for bit what the passes give run one by one over the
    whole state (Gaussian inputs, normalised)."""
    say("block chunks %s n=%d batch=%d split=%s" % (dtype, n, batch, split))
    tdt = torch.float32 if dtype == "f32" else torch.float64
    plan = qse.Plan(n, dtype, split=split)
    cp, bb, bl = plan.call_schedule(batch)
    assert 2 <= cp < plan.num_passes and bb < n and (batch << (n - bb)) > bl
    g = torch.Generator(device="cuda").manual_seed(n)
    re = torch.randn(batch, 1 << n, generator=g, device="cuda", dtype=tdt)
    im = torch.randn(batch, 1 << n, generator=g, device="cuda", dtype=tdt)
    r1, i1 = re.clone(), im.clone()
    plan.execute(re, im, normalize=True)
    for i in range(plan.num_passes):
        plan.execute_pass(i, r1, i1, normalize=True)
    torch.cuda.synchronize()
    assert torch.equal(re, r1) and torch.equal(im, i1)
    if n > 27:
        return
    # and against the oracle on one sampled vector
    v = batch - 1
    x_re, x_im = r1[v].cpu().numpy(), i1[v].cpu().numpy()
    del r1, i1
    torch.cuda.empty_cache()
    g = torch.Generator(device="cuda").manual_seed(n)
    o_re = torch.randn(batch, 1 << n, generator=g, device="cuda", dtype=tdt)[v].cpu().numpy()
    o_im = torch.randn(batch, 1 << n, generator=g, device="cuda", dtype=tdt)[v].cpu().numpy()
    assert_close(dtype, n, o_re, o_im, x_re, x_im)


def _parity(t):
    """popcount(t) mod 2 for a non-negative int64 tensor (below 2^32)."""
    for sh in (16, 8, 4, 2, 1):
        t = t ^ (t >> sh)
    return t & 1


@pytest.mark.parametrize("dtype,n", [("f32", 30), ("f64", 29), ("f64", 30)])
def test_largest_n_closed_form(dtype, n):
    """The largest n each dtype supports: x = e_j + 2 e_k (re) and e_k - e_j
    (im) transform to (-1)^popcount(i AND j) + 2 (-1)^popcount(i AND k) and
    so on, checked for all 2^n outputs on the device (exact)."""
    say("largest n %s n=%d" % (dtype, n))
    tdt = torch.float32 if dtype == "f32" else torch.float64
    N = 1 << n
    j, k = 0x2AAAAAAA & (N - 1), 0x15555555 & (N - 1) | (1 << (n - 1))
    re = torch.zeros(1, N, dtype=tdt, device="cuda")
    im = torch.zeros(1, N, dtype=tdt, device="cuda")
    re[0, j] = 1.0
    re[0, k] = 2.0
    im[0, k] = 1.0
    im[0, j] = -1.0
    plan = qse.Plan(n, dtype)
    plan.execute(re, im, normalize=False)
    torch.cuda.synchronize()
    i = torch.arange(N, device="cuda", dtype=torch.int64)
    sj = (1 - 2 * _parity(i & j)).to(tdt)
    sk = (1 - 2 * _parity(i & k)).to(tdt)
    del i
    assert torch.equal(re[0], sj + 2 * sk)
    assert torch.equal(im[0], sk - sj)
    del re, im, sj, sk
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,n,batch", [("f32", 4, 1 << 24), ("f64", 3, 1 << 23),
                                           ("f32", 10, (1 << 16) + 3), ("f32", 14, 2048),
                                           ("f32", 14, 2049), ("f64", 13, 2048),
                                           ("f64", 13, 2051)])
def test_large_batch_one_pass(dtype, n, batch):
    """One-pass plans (the wave-tile kernel by default) at the largest
    batches a 1-2 GiB state holds, ragged in the last case, and the
    12-vector-bit plans on either side of their 256 MiB switch between two
    tilings: sampled vectors exactly against the oracle, and every vector
    through the exact normalised involution (integer inputs, even n:
    H H / 2^n = I)."""
    say("large batch %s n=%d batch=%d" % (dtype, n, batch))
    tdt = torch.float32 if dtype == "f32" else torch.float64
    g = torch.Generator(device="cuda").manual_seed(4242 + n)
    re = torch.randint(-8, 9, (batch, 1 << n), generator=g, device="cuda").to(tdt)
    im = torch.randint(-8, 9, (batch, 1 << n), generator=g, device="cuda").to(tdt)
    plan = qse.Plan(n, dtype)
    if n - (2 if dtype == "f32" else 1) == 12:
        resident = batch * (2 << n) * (4 if dtype == "f32" else 8) <= 256 << 20
        assert plan.pass_config(0, batch)["eb"] == (3 if resident else 2)
    rows = [0, 1, batch // 3, batch - 1]
    re0, im0 = re[rows].cpu().numpy(), im[rows].cpu().numpy()
    ore, oim = re.clone(), im.clone()
    plan.execute(re, im, normalize=False)
    torch.cuda.synchronize()
    assert_exact(re[rows].cpu().numpy(), re0, n, False)
    assert_exact(im[rows].cpu().numpy(), im0, n, False)
    if n % 2 == 0:
        re.copy_(ore)
        im.copy_(oim)
        plan.execute(re, im, normalize=True)
        plan.execute(re, im, normalize=True)
        torch.cuda.synchronize()
        assert torch.equal(re, ore) and torch.equal(im, oim)
    del re, im, ore, oim
    torch.cuda.empty_cache()


# ---- API behaviour on the device ----------------------------------------------

def test_real_only_transform():
    say("real only")
    n = 12
    re = ints((4, 1 << n), 7, np.float32)
    tre = to_dev(re)
    qse.Plan(n, "f32").execute(tre, None, normalize=False)
    torch.cuda.synchronize()
    assert_exact(tre.cpu().numpy(), re, n, False)


def test_non_default_stream_and_determinism():
    say("stream + determinism")
    n = 20
    w = workloads.custom(n, 4, "f32", "gauss", True, seed=11)
    re, im = workloads.gen(w)
    s = torch.cuda.Stream()
    plan = qse.Plan(n, "f32")
    a_re, a_im = to_dev(re), to_dev(im)
    b_re, b_im = to_dev(re), to_dev(im)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        plan.execute(a_re, a_im, normalize=True)
    plan.execute(b_re, b_im, normalize=True, stream=s)
    s.synchronize()
    assert torch.equal(a_re, b_re) and torch.equal(a_im, b_im)
    assert_close("f32", n, re, im, a_re.cpu().numpy(), a_im.cpu().numpy())


@pytest.mark.parametrize("n,batch", [(10, 256), (12, 256), (14, 256), (20, 4)])
def test_repeated_calls_bit_identical(n, batch):
    """The fp32 lane stages on lane bits 0 and 1 are hand-written DPP
    multiply-adds whose wait states are set by hand.  Twenty calls on the
    same Gaussian input, with many waves resident, must give the same bits
    every time (a missed wait state would show as a timing-dependent
    result), and the first must match the oracle."""
    say("repeat n=%d batch=%d" % (n, batch))
    w = workloads.custom(n, batch, "f32", "gauss", True, seed=12_000 + n)
    re, im = workloads.gen(w)
    plan = qse.Plan(n, "f32")
    src_re, src_im = to_dev(re), to_dev(im)
    first = None
    for rep in range(20):
        t_re, t_im = src_re.clone(), src_im.clone()
        plan.execute(t_re, t_im, normalize=True)
        if first is None:
            torch.cuda.synchronize()
            first = (t_re, t_im)
            assert_close("f32", n, re, im, t_re.cpu().numpy(), t_im.cpu().numpy())
        else:
            assert torch.equal(t_re, first[0]) and torch.equal(t_im, first[1]), "call %d" % rep


def test_one_plan_from_several_threads_and_streams():
    """One plan used at once from four host threads, each on its own
    stream and buffers (ctypes releases the GIL during the call): every
    result equals the single-threaded one bit for bit."""
    import threading
    say("threads + streams")
    n = 18
    w = workloads.custom(n, 6, "f32", "gauss", True, seed=12)
    re, im = workloads.gen(w)
    plan = qse.Plan(n, "f32")
    ref_re, ref_im = to_dev(re), to_dev(im)
    plan.execute(ref_re, ref_im, normalize=True)
    torch.cuda.synchronize()
    bufs = [(to_dev(re), to_dev(im), torch.cuda.Stream()) for _ in range(4)]
    torch.cuda.synchronize()
    errors = []

    def worker(b_re, b_im, stream):
        try:
            for _ in range(8):   # an even count: back to the input ...
                plan.execute(b_re, b_im, normalize=True, stream=stream)
            plan.execute(b_re, b_im, normalize=True, stream=stream)   # ... then once more
        except Exception as e:   # reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=b) for b in bufs]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for b_re, b_im, _ in bufs:
        assert_close("f32", n, re, im, b_re.cpu().numpy(), b_im.cpu().numpy())
        # nine calls differ from one only by rounding
        assert torch.allclose(b_re, ref_re, atol=1e-5) and torch.allclose(b_im, ref_im, atol=1e-5)
    # identical inputs and call sequences give identical results
    for b_re, b_im, _ in bufs[1:]:
        assert torch.equal(b_re, bufs[0][0]) and torch.equal(b_im, bufs[0][1])


@pytest.mark.parametrize("n,batch,dtype", [(12, 5, "f32"), (20, 4, "f32"), (22, 2, "f64"),
                                           (24, 3, "f64"), (27, 1, "f32")])
def test_hip_graph_capture_and_replay(n, batch, dtype):
    """fwt_execute captured into a HIP graph (torch's default capture mode)
    and replayed three times, with other eager work and synchronisations
    between the replays: every replay equals the eager call bit for bit.
    The library records kernel launches only (no memset nodes).  The last
    two cases capture chunked schedules: chunks of vectors (fp64 n=24) and
    of sub-vector blocks (fp32 n=27)."""
    say("graph %s n=%d batch=%d" % (dtype, n, batch))
    w = workloads.custom(n, batch, dtype, "gauss", True, seed=31)
    re0, im0 = workloads.gen(w)
    plan = qse.Plan(n, dtype)
    e_re, e_im = to_dev(re0), to_dev(im0)
    plan.execute(e_re, e_im, normalize=True)
    torch.cuda.synchronize()
    x_re, x_im = to_dev(re0), to_dev(im0)
    g_re, g_im = torch.empty_like(x_re), torch.empty_like(x_im)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        fn = plan.bind(g_re, g_im, normalize=True, stream=s)
        g_re.copy_(x_re)
        g_im.copy_(x_im)
        fn()                         # warm-up outside the capture
        s.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            fn()
    for rep in range(3):
        g_re.copy_(x_re)
        g_im.copy_(x_im)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g_re, e_re) and torch.equal(g_im, e_im), "replay %d" % rep
        junk = torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")
        torch.cuda.synchronize()
        del junk


def test_involution_normalised():
    say("involution")
    for n, dtype in ((13, "f32"), (20, "f32"), (17, "f64")):
        w = workloads.custom(n, 2, dtype, "gauss", True, seed=n)
        re, im = workloads.gen(w)
        tre, tim = to_dev(re), to_dev(im)
        plan = qse.Plan(n, dtype)
        plan.execute(tre, tim, True)
        plan.execute(tre, tim, True)
        torch.cuda.synchronize()
        tol = 2 * TOL[dtype]
        assert np.abs(tre.cpu().numpy() - re).max() <= tol
        assert np.abs(tim.cpu().numpy() - im).max() <= tol


def test_guard_regions_untouched():
    say("guard regions")
    pad = 1024
    for n, dtype, batch in ((12, "f32", 3), (20, "f32", 2), (14, "f64", 3), (22, "f64", 1)):
        npd = np.float32 if dtype == "f32" else np.float64
        N = 1 << n
        sentinel = 12345.0
        bufs = [torch.full((pad + batch * N + pad,), sentinel, dtype=torch.float32
                           if dtype == "f32" else torch.float64, device="cuda") for _ in range(2)]
        re = ints((batch, N), n, npd)
        im = ints((batch, N), n + 1, npd)
        bufs[0][pad:pad + batch * N] = to_dev(re.ravel())
        bufs[1][pad:pad + batch * N] = to_dev(im.ravel())
        qse.Plan(n, dtype).execute(bufs[0][pad:pad + batch * N], bufs[1][pad:pad + batch * N],
                                   normalize=False)
        torch.cuda.synchronize()
        for t, x in zip(bufs, (re, im)):
            h = t.cpu().numpy()
            assert (h[:pad] == sentinel).all() and (h[pad + batch * N:] == sentinel).all()
            assert_exact(h[pad:pad + batch * N].reshape(batch, N), x, n, False)


def _alloc_range(ptr):
    hip = ctypes.CDLL("libamdhip64.so")
    base, size = ctypes.c_void_p(), ctypes.c_size_t()
    st = hip.hipMemGetAddressRange(ctypes.byref(base), ctypes.byref(size), ctypes.c_void_p(ptr))
    assert st == 0
    return base.value, size.value


def test_validation_on_device_memory():
    say("validation")
    n = 10
    N = 1 << n
    plan = qse.Plan(n, "f32")
    re = torch.zeros(4 * N, device="cuda")
    im = torch.zeros(4 * N, device="cuda")
    assert plan.check_raw(4, re.data_ptr(), im.data_ptr()) == qse.FWT_OK
    host = np.zeros(4 * N, np.float32)
    assert plan.check_raw(4, host.ctypes.data, im.data_ptr()) == qse.FWT_EINVAL
    base, size = _alloc_range(re.data_ptr())
    too_many = (base + size - re.data_ptr()) // (4 * N) + 1
    assert plan.check_raw(too_many, re.data_ptr(), None) == qse.FWT_EINVAL
    # fwt_execute runs the same validation first, so it rejects before launching
    assert plan.execute_raw(too_many, re.data_ptr(), 0, 1) == qse.FWT_EINVAL
    with pytest.raises(qse.FwtError):
        plan.execute(re, re)   # same buffer twice
    assert plan.execute_raw(0, re.data_ptr(), im.data_ptr(), 1) == qse.FWT_OK


def test_timed_passes_follow_the_chunk_schedule():
    """Running every pass of every chunk with fwt_execute_pass_timed (the
    benchmark's per-kernel timing) is exactly fwt_execute."""
    say("timed passes")
    n, batch = 20, 40
    plan = qse.Plan(n, "f32")
    cv = plan.chunk_vectors(batch, True)
    assert 0 < cv < batch
    re = ints((batch, 1 << n), 91, np.float32)
    im = ints((batch, 1 << n), 92, np.float32)
    tre, tim = to_dev(re), to_dev(im)
    times = []
    for c0 in range(0, batch, cv):
        sl = slice(c0, min(batch, c0 + cv))
        for i in range(plan.num_passes):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            plan.execute_pass_timed(i, tre[sl], tim[sl], a, b, normalize=False)
            times.append((a, b))
    torch.cuda.synchronize()
    assert all(a.elapsed_time(b) > 0 for a, b in times)
    gre, gim = run(plan, re, im, False)
    assert np.array_equal(tre.cpu().numpy(), gre) and np.array_equal(tim.cpu().numpy(), gim)
    assert_exact(gre[: 3], re[: 3], n, False)


ABLATION_KINDS = {"stagewise": qse.ABLATION_STAGEWISE, "popc_gemm": qse.ABLATION_POPC_GEMM,
                  "mfma": qse.ABLATION_MFMA, "mfma_transpose": qse.ABLATION_MFMA_TRANSPOSE}


@pytest.mark.parametrize("kind", ["stagewise", "popc_gemm", "mfma"])
@pytest.mark.parametrize("dtype,n,batch", [("f32", 2, 5), ("f32", 5, 3), ("f32", 10, 8), ("f32", 13, 2),
                                           ("f32", 14, 3), ("f64", 1, 4), ("f64", 2, 3), ("f64", 9, 5),
                                           ("f64", 14, 2), ("f32", 17, 1)])
def test_integer_ablations(kind, dtype, n, batch):
    """The pages' designs (one launch per stage; popcount GEMM + transposes;
    H_16 blocks on the matrix cores) compute exactly the same transform.
    Below their smallest size (the scaffold: n < 2; the matrix-core row
    kernel: n < 8) they refuse with FWT_EUNSUPPORTED and leave the data as
    it was."""
    k = ABLATION_KINDS[kind]
    say("ablation %s %s n=%d batch=%d" % (kind, dtype, n, batch))
    npd = np.float32 if dtype == "f32" else np.float64
    re = ints((batch, 1 << n), 99_000 + n, npd)
    im = ints((batch, 1 << n), 99_500 + n, npd)
    if (kind == "popc_gemm" and n < 2) or (kind == "mfma" and n < 8):
        tre, tim = to_dev(re), to_dev(im)
        with pytest.raises(qse.FwtError) as ei:
            qse.ablation_execute(k, tre, tim, n=n, normalize=False, workspace=None)
        assert ei.value.status == qse.FWT_EUNSUPPORTED
        torch.cuda.synchronize()
        assert np.array_equal(tre.cpu().numpy(), re) and np.array_equal(tim.cpu().numpy(), im)
        return
    for normalize in (False, True):
        if normalize and n % 2:
            continue
        tre, tim = to_dev(re), to_dev(im)
        wsb = qse.ablation_workspace(k, batch, n, dtype, True)
        ws = torch.empty(max(wsb, 16) // 4, dtype=torch.float32, device="cuda") if wsb else None
        qse.ablation_execute(k, tre, tim, n=n, normalize=normalize, workspace=ws)
        torch.cuda.synchronize()
        assert_exact(tre.cpu().numpy(), re, n, normalize)
        assert_exact(tim.cpu().numpy(), im, n, normalize)


# Matrix-core ablation at every row width it has (8..15 low bits fp32,
# 8..14 fp64; 1024-thread workgroups from 13), with ragged last workgroups
# (11 bits: 2 tiles per workgroup, odd tile counts), one and two column
# passes (n = 26: 10 | 8 | 8) and a state larger than one cache chunk (fp32
# n = 20, 80 vectors).
@pytest.mark.parametrize("dtype,n,batch", [("f32", 8, 7), ("f64", 8, 3), ("f32", 11, 33),
                                           ("f64", 11, 5), ("f32", 12, 3), ("f64", 12, 2),
                                           ("f32", 13, 3), ("f64", 13, 2), ("f32", 14, 2),
                                           ("f64", 14, 3), ("f32", 15, 2), ("f32", 16, 3),
                                           ("f64", 21, 1), ("f32", 26, 1), ("f32", 20, 80)])
def test_integer_mfma_ablation(dtype, n, batch):
    say("ablation mfma %s n=%d batch=%d" % (dtype, n, batch))
    npd = np.float32 if dtype == "f32" else np.float64
    re = ints((batch, 1 << n), 98_000 + n, npd)
    im = ints((batch, 1 << n), 98_500 + n, npd)
    normalize = n % 2 == 0
    tre, tim = to_dev(re), to_dev(im)
    qse.ablation_execute(qse.ABLATION_MFMA, tre, tim, n=n, normalize=normalize)
    torch.cuda.synchronize()
    assert_exact(tre.cpu().numpy(), re, n, normalize)
    assert_exact(tim.cpu().numpy(), im, n, normalize)


# INT8 / CRT ablation (fp64): every pass shape it plans (row pass only,
# one and two column passes of 1..9 bits), ragged batches, real-only.
@pytest.mark.parametrize("n,batch", [(5, 3), (7, 5), (9, 2), (10, 1), (11, 3), (12, 2), (13, 1),
                                     (16, 3), (19, 1), (20, 2), (21, 1), (24, 1)])
def test_integer_ozaki_ablation(n, batch):
    say("ablation ozaki n=%d batch=%d" % (n, batch))
    re = ints((batch, 1 << n), 91_000 + n, np.float64)
    im = ints((batch, 1 << n), 91_500 + n, np.float64)
    for normalize in ((False, True) if n % 2 == 0 else (False,)):
        tre, tim = to_dev(re), to_dev(im)
        wsb = qse.ablation_workspace(qse.ABLATION_OZAKI, batch, n, "f64", True)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        qse.ablation_execute(qse.ABLATION_OZAKI, tre, tim, n=n, normalize=normalize, workspace=ws)
        torch.cuda.synchronize()
        assert_exact(tre.cpu().numpy(), re, n, normalize)
        assert_exact(tim.cpu().numpy(), im, n, normalize)
    # real-only
    tre = to_dev(re)
    wsb = qse.ablation_workspace(qse.ABLATION_OZAKI, batch, n, "f64", False)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    qse.ablation_execute(qse.ABLATION_OZAKI, tre, None, n=n, normalize=False, workspace=ws)
    torch.cuda.synchronize()
    assert_exact(tre.cpu().numpy(), re, n, False)


@pytest.mark.parametrize("n,batch", [(13, 3), (20, 2), (24, 1)])
def test_gaussian_ozaki_ablation(n, batch):
    """Gaussian states, with per-vector scales far apart (1e-100, 1, 1e100
    and an all-zero vector): each vector's own power-of-two scale keeps the
    fp64 tolerance.  (Scales stay where the squared norm of the bound does
    not underflow.)"""
    say("ablation ozaki gauss n=%d batch=%d" % (n, batch))
    w = workloads.custom(n, batch, "f64", "gauss", True, seed=300 + n)
    re, im = workloads.gen(w)
    re, im = re.reshape(batch, -1).copy(), im.reshape(batch, -1).copy()
    scales = [1e-100, 1.0, 1e100][:batch]
    for b, sc in enumerate(scales):
        re[b] *= sc
        im[b] *= sc
    if batch >= 3:
        re[1] = 0.0
        im[1] = 0.0
    tre, tim = to_dev(re), to_dev(im)
    wsb = qse.ablation_workspace(qse.ABLATION_OZAKI, batch, n, "f64", True)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    qse.ablation_execute(qse.ABLATION_OZAKI, tre, tim, n=n, normalize=True, workspace=ws)
    torch.cuda.synchronize()
    assert_close("f64", n, re, im, tre.cpu().numpy(), tim.cpu().numpy())


@pytest.mark.parametrize("dtype,n,batch", [("f32", 9, 5), ("f32", 20, 3), ("f64", 13, 3),
                                           ("f64", 24, 1)])
def test_mfma_path_plan(dtype, n, batch):
    """A FWT_PATH_MFMA_ABLATION plan through fwt_execute, and pass by pass
    through the dispatch-timed entry, exactly."""
    say("mfma path %s n=%d batch=%d" % (dtype, n, batch))
    npd = np.float32 if dtype == "f32" else np.float64
    re = ints((batch, 1 << n), 93_000 + n, npd)
    im = ints((batch, 1 << n), 93_500 + n, npd)
    plan = qse.Plan(n, dtype, path=qse.PATH_MFMA_ABLATION)
    assert plan.pass_config(0)["kind"] == "mfma"
    normalize = n % 2 == 0
    gre, gim = run(plan, re, im, normalize)
    assert_exact(gre, re, n, normalize)
    assert_exact(gim, im, n, normalize)
    tre, tim = to_dev(re), to_dev(im)
    evs = []
    for i in range(plan.num_passes):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        plan.execute_pass_timed(i, tre, tim, a, b, normalize=normalize)
        evs.append((a, b))
    torch.cuda.synchronize()
    assert all(a.elapsed_time(b) > 0 for a, b in evs)
    assert np.array_equal(tre.cpu().numpy(), gre) and np.array_equal(tim.cpu().numpy(), gim)


@pytest.mark.parametrize("kind", ["stagewise", "popc_gemm", "mfma", "mfma_transpose"])
def test_gaussian_ablations_n20(kind):
    k = ABLATION_KINDS[kind]
    say("ablation gauss %s n=20" % kind)
    w = workloads.custom(20, 2, "f32", "gauss", True, seed=77)
    re, im = workloads.gen(w)
    tre, tim = to_dev(re), to_dev(im)
    wsb = qse.ablation_workspace(k, 2, 20, "f32", True)
    ws = torch.empty(wsb // 4, device="cuda") if wsb else None
    qse.ablation_execute(k, tre, tim, n=20, normalize=True, workspace=ws)
    torch.cuda.synchronize()
    assert_close("f32", 20, re, im, tre.cpu().numpy(), tim.cpu().numpy())


# Matrix-core block products on both factors with the transposed staging
# buffer: every split n/2 | n - n/2 from 8 | 8 to the widest (15 | 15 fp32,
# 14 | 14 fp64), odd n, several vectors.
@pytest.mark.parametrize("dtype,n,batch", [("f32", 16, 3), ("f32", 17, 2), ("f32", 20, 2),
                                           ("f32", 23, 1), ("f64", 16, 3), ("f64", 19, 2),
                                           ("f64", 23, 1)])
def test_integer_mfma_transpose_ablation(dtype, n, batch):
    say("ablation mfma+transpose %s n=%d batch=%d" % (dtype, n, batch))
    k = qse.ABLATION_MFMA_TRANSPOSE
    npd = np.float32 if dtype == "f32" else np.float64
    # n >= 23: inputs in {-1, 0, 1} keep every partial sum an exact integer
    lo, hi = (-8, 9) if n < 23 else (-1, 2)
    rng = np.random.default_rng(98_000 + n)
    re = rng.integers(lo, hi, size=(batch, 1 << n)).astype(npd)
    im = rng.integers(lo, hi, size=(batch, 1 << n)).astype(npd)
    for normalize in (False, True):
        if normalize and (n % 2 or n >= 23):
            continue
        tre, tim = to_dev(re), to_dev(im)
        wsb = qse.ablation_workspace(k, batch, n, dtype, True)
        ws = torch.empty(wsb // 4, dtype=torch.float32, device="cuda")
        qse.ablation_execute(k, tre, tim, n=n, normalize=normalize, workspace=ws)
        torch.cuda.synchronize()
        assert_exact(tre.cpu().numpy(), re, n, normalize)
        assert_exact(tim.cpu().numpy(), im, n, normalize)
        del ws


@pytest.mark.parametrize("dtype,n", [("f32", 30), ("f64", 28)])
def test_mfma_transpose_ablation_widest(dtype, n):
    """The widest split (15 | 15 fp32, 14 | 14 fp64): a two-hot input
    against its closed form at all 2^n outputs, on the device (exact)."""
    say("ablation mfma+transpose widest %s n=%d" % (dtype, n))
    tdt = torch.float32 if dtype == "f32" else torch.float64
    N = 1 << n
    j, k = 0x2AAAAAAA & (N - 1), 0x15555555 & (N - 1) | (1 << (n - 1))
    re = torch.zeros(1, N, dtype=tdt, device="cuda")
    im = torch.zeros(1, N, dtype=tdt, device="cuda")
    re[0, j] = 1.0
    re[0, k] = 2.0
    im[0, k] = 1.0
    im[0, j] = -1.0
    kind = qse.ABLATION_MFMA_TRANSPOSE
    ws = torch.empty(qse.ablation_workspace(kind, 1, n, dtype, True) // 4, device="cuda")
    qse.ablation_execute(kind, re, im, n=n, normalize=False, workspace=ws)
    torch.cuda.synchronize()
    del ws
    i = torch.arange(N, device="cuda", dtype=torch.int64)
    sj = (1 - 2 * _parity(i & j)).to(tdt)
    sk = (1 - 2 * _parity(i & k)).to(tdt)
    del i
    assert torch.equal(re[0], sj + 2 * sk)
    assert torch.equal(im[0], sk - sj)
    del re, im, sj, sk
    torch.cuda.empty_cache()


def test_bound_call_keeps_its_plan_alive():
    """A callable from Plan.bind stays valid after the Plan object itself
    goes out of scope."""
    say("bind lifetime")
    import gc
    n = 10
    re = ints((4, 1 << n), 5, np.float32)
    tre = to_dev(re)
    step = qse.Plan(n, "f32").bind(tre, None, normalize=False)
    gc.collect()
    torch.cuda.synchronize()
    assert np.array_equal(tre.cpu().numpy(), re)     # binding runs nothing
    step()
    torch.cuda.synchronize()
    assert_exact(tre.cpu().numpy(), re, n, False)


def test_bound_call_keeps_its_tensors_alive():
    """The callable holds the bound tensors: when the caller drops its own
    references, torch's caching allocator cannot hand their memory to a new
    tensor, so a later call transforms the bound data and nothing else."""
    say("bind keeps tensors")
    import gc
    import weakref
    n = 10
    re = ints((4, 1 << n), 6, np.float32)
    im = ints((4, 1 << n), 7, np.float32)
    tre, tim = to_dev(re), to_dev(im)
    step = qse.Plan(n, "f32").bind(tre, tim, normalize=False)
    ref_re, ref_im = weakref.ref(tre), weakref.ref(tim)
    del tre, tim
    gc.collect()
    assert ref_re() is not None and ref_im() is not None
    other = torch.full((4, 1 << n), 3.0, device="cuda")   # same size, allocated after
    step()
    torch.cuda.synchronize()
    assert torch.equal(other, torch.full_like(other, 3.0))
    assert_exact(ref_re().cpu().numpy(), re, n, False)
    assert_exact(ref_im().cpu().numpy(), im, n, False)
    del step
    gc.collect()
    assert ref_re() is None and ref_im() is None          # released with the callable


def test_stream_copy():
    say("stream copy")
    src = torch.randn(3 * 2**20 + 12, device="cuda")
    dst = torch.empty_like(src)
    qse.stream_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
