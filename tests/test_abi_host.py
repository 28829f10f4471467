"""Host-side tests of the C ABI (no GPU): the library loads, exports every
declared symbol, plans split n as documented, and fwt_execute rejects bad
arguments before it makes any HIP call."""
import ctypes
import os
import re

import pytest

import quantum_state_encoding_amd as qse

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fwt.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fwt_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(qse.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_strerror_covers_every_status(lib):
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert lib.fwt_strerror(st).decode() != "unknown status"
    assert lib.fwt_strerror(7).decode() == "unknown status"


def _create(lib, n, dtype=0, path=0):
    h = ctypes.c_void_p()
    st = lib.fwt_plan_create(ctypes.byref(h), n, dtype, path)
    return st, h


def _split(lib, n, dtype, bits, eb=None, gbits=None, phases=None, pipe=None, wave=None):
    h = ctypes.c_void_p()
    arr = (ctypes.c_int * len(bits))(*bits)
    knobs = {"eb": eb, "gbits": gbits, "phases": phases, "pipe": pipe, "wave": wave}
    if all(v is None for v in knobs.values()):
        st = lib.fwt_plan_create_split(ctypes.byref(h), n, dtype, len(bits), arr)
    else:
        tun = (qse.PassTuning * len(bits))()
        for i in range(len(bits)):
            for name, vals in knobs.items():
                setattr(tun[i], name, -1 if vals is None else vals[i])
        st = lib.fwt_plan_create_tuned(ctypes.byref(h), n, dtype, len(bits), arr, tun)
    if st == 0:
        lib.fwt_plan_destroy(h)
    return st


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_default_plans_cover_all_bits(dtype, lib):
    nmax = 30
    for n in range(0, nmax + 1):
        p = qse.Plan(n, dtype)
        bits = p.pass_bits
        assert sum(bits) == n
        assert p.num_passes == len(bits)
        if n <= 24:
            assert p.num_passes <= 2, (n, bits)
        p.close()


def test_plan_shapes_of_the_workloads(lib):
    assert qse.Plan(10, "f32").pass_bits == [10]
    assert qse.Plan(12, "f32").pass_bits == [12]
    assert qse.Plan(14, "f32").pass_bits == [14]
    assert qse.Plan(14, "f32", split=(7, 7)).pass_bits == [7, 7]
    assert qse.Plan(20, "f32").pass_bits == [12, 8]
    assert qse.Plan(24, "f64").pass_bits == [14, 10]


def test_default_splits(lib):
    # two passes: a 9-bit column factor, a row pass of >= 8 vector bits (not
    # 9) and at most one tile; column factors up to 11 bits; then 3 passes
    want = {"f32": {16: [10, 6], 17: [10, 7], 18: [10, 8], 19: [10, 9], 20: [12, 8],
                    21: [12, 9], 22: [13, 9], 23: [14, 9], 24: [15, 9], 25: [15, 10],
                    26: [15, 11], 27: [10, 9, 8], 30: [10, 10, 10]},
            "f64": {15: [9, 6], 18: [9, 9], 19: [11, 8], 20: [11, 9], 21: [12, 9],
                    22: [13, 9], 23: [14, 9], 24: [14, 10], 25: [14, 11], 26: [10, 8, 8],
                    29: [10, 10, 9], 30: [10, 10, 10]}}
    for dtype, table in want.items():
        for n, bits in table.items():
            assert qse.Plan(n, dtype).pass_bits == bits, (dtype, n)


def test_chunk_schedule(lib):
    p20 = qse.Plan(20, "f32")
    assert p20.chunk_vectors(256, True) == 32       # 8 MiB per complex vector, 256 MiB chunks
    assert p20.chunk_vectors(256, False) == 64
    assert p20.chunk_vectors(32, True) == 0         # fits: one chunk
    assert qse.Plan(24, "f64").chunk_vectors(16, True) == 1
    assert qse.Plan(12, "f32").chunk_vectors(10**6, True) == 0   # single pass: never chunked
    # the whole schedule: (chunked passes, log2 elements per block, blocks per chunk)
    assert p20.call_schedule(256) == (2, 20, 32)
    assert p20.call_schedule(32) == (0, 20, 0)
    assert qse.Plan(24, "f64").call_schedule(16) == (2, 24, 1)
    # one vector above 256 MiB: the leading passes run on chunks of blocks
    p27 = qse.Plan(27, "f32")
    assert p27.pass_bits == [10, 9, 8]
    assert p27.call_schedule(2) == (2, 19, 64) and p27.chunk_vectors(2) == 0
    assert p27.call_schedule(2, False) == (2, 19, 128)
    assert qse.Plan(26, "f64").call_schedule(2) == (2, 18, 64)
    assert qse.Plan(30, "f32").call_schedule(1) == (2, 20, 32)
    assert qse.Plan(30, "f64").call_schedule(1) == (2, 20, 16)
    assert qse.Plan(28, "f32", split=(7, 7, 7, 7)).call_schedule(1) == (3, 21, 16)
    # two-pass plans with such vectors keep one vector per chunk
    assert qse.Plan(26, "f32").call_schedule(4) == (2, 26, 1)
    assert qse.Plan(26, "f32").chunk_vectors(4) == 1
    for pl in (p20, p27):
        for batch in (1, 3, 64, 1000):
            cp, bb, bl = pl.call_schedule(batch)
            cv = pl.chunk_vectors(batch)
            assert cv == (bl if cp and bb == pl.n else 0)
    assert qse.Plan(14, "f32", path=qse.PATH_MULTIPASS).pass_bits == [7, 7]
    assert qse.Plan(15, "f32", path=qse.PATH_SINGLE_BLOCK).pass_bits == [15]


def test_plan_create_errors(lib):
    assert _create(lib, -1)[0] == qse.FWT_EINVAL
    assert _create(lib, 31)[0] == qse.FWT_EINVAL
    assert _create(lib, 10, dtype=2)[0] == qse.FWT_EINVAL
    assert _create(lib, 10, path=9)[0] == qse.FWT_EINVAL
    assert _create(lib, 7, path=qse.PATH_MFMA_ABLATION)[0] == qse.FWT_EUNSUPPORTED
    assert _create(lib, 30, 1, qse.PATH_MFMA_ABLATION)[0] == qse.FWT_EUNSUPPORTED
    assert _create(lib, 16, 0, qse.PATH_SINGLE_BLOCK)[0] == qse.FWT_EUNSUPPORTED
    assert _create(lib, 15, 1, qse.PATH_SINGLE_BLOCK)[0] == qse.FWT_EUNSUPPORTED
    st, h = _create(lib, 30, 1)      # fp64 n = 30: its top pass spans 8 GiB per tile
    assert st == qse.FWT_OK
    lib.fwt_plan_destroy(h)
    assert lib.fwt_plan_create(None, 10, 0, 0) == qse.FWT_EINVAL


def test_split_validation(lib):
    assert _split(lib, 10, 0, [5, 5]) == 0
    assert _split(lib, 10, 0, [2, 8]) == 0
    assert _split(lib, 10, 0, [3, 3, 4]) == 0
    assert _split(lib, 10, 0, [4, 4]) == qse.FWT_EINVAL        # sum != n
    assert _split(lib, 10, 0, [1, 9]) == qse.FWT_EINVAL        # fp32 row pass needs 2 bits
    assert _split(lib, 10, 1, [1, 9]) == 0                     # fp64 needs 1
    assert _split(lib, 20, 0, [7, 13]) == qse.FWT_EINVAL       # column pass > 12 bits
    assert _split(lib, 20, 0, [16, 4]) == qse.FWT_EINVAL       # row pass > 15 bits
    assert _split(lib, 10, 0, [5, 0, 5]) == qse.FWT_EINVAL     # empty factor
    assert _split(lib, 10, 0, [2, 2, 2, 2, 2]) == qse.FWT_EINVAL  # > 4 passes
    h = ctypes.c_void_p()
    assert lib.fwt_plan_create_split(ctypes.byref(h), 10, 0, 0, None) == qse.FWT_EINVAL
    assert lib.fwt_plan_create_split(ctypes.byref(h), 10, 0, 2, None) == qse.FWT_EINVAL


def test_tuned_validation(lib):
    assert _split(lib, 16, 0, [8, 8], eb=[3, 4], gbits=[-1, 2]) == 0
    assert _split(lib, 16, 0, [8, 8], eb=[5, 3], gbits=[0, 4]) == 0
    assert _split(lib, 16, 0, [8, 8], eb=[9, 4]) == qse.FWT_EINVAL      # eb > kr
    assert _split(lib, 16, 0, [8, 8], gbits=[1, 2]) == qse.FWT_EINVAL   # row pass G = 1
    assert _split(lib, 16, 0, [8, 8], gbits=[0, 7]) == qse.FWT_EINVAL   # too many groups
    assert _split(lib, 12, 0, [2, 10], gbits=[0, 1]) == qse.FWT_EINVAL  # only 1 group in a row
    assert _split(lib, 24, 1, [12, 12], gbits=[0, 3]) == qse.FWT_EINVAL  # tile > 160 KiB
    assert _split(lib, 24, 1, [14, 10], gbits=[-1, 3], phases=[-1, 1]) == 0
    assert _split(lib, 24, 1, [14, 10], gbits=[-1, 3], phases=[-1, 2]) == 0
    assert _split(lib, 24, 1, [14, 10], gbits=[-1, 3], phases=[-1, 0]) == 0   # 128 KiB, 1 tile/CU
    assert _split(lib, 24, 1, [14, 10], gbits=[-1, 2], phases=[-1, 3]) == qse.FWT_EINVAL
    assert _split(lib, 20, 0, [13, 7], phases=[-1, 1]) == qse.FWT_EINVAL    # < 9 column bits
    assert _split(lib, 20, 0, [13, 7], phases=[1, -1]) == qse.FWT_EINVAL    # row pass
    assert _split(lib, 24, 1, [14, 10], pipe=[1, 0]) == 0
    assert _split(lib, 24, 1, [14, 10], pipe=[0, 1]) == 0
    assert _split(lib, 24, 1, [14, 10], pipe=[2, 0]) == qse.FWT_EINVAL
    assert _split(lib, 12, 0, [2, 10], pipe=[1, -1]) == qse.FWT_EUNSUPPORTED  # tiny tile
    # wave-tile passes: lane bits are limited to 6 - gbits
    assert _split(lib, 12, 0, [12], wave=[1]) == 0                 # kr 10 = 4 regs + 6 lanes
    assert _split(lib, 13, 0, [13], wave=[1]) == 0                 # kr 11 = 5 + 6
    assert _split(lib, 14, 0, [14], wave=[1]) == qse.FWT_EINVAL    # kr 12 > 11
    assert _split(lib, 12, 0, [12], eb=[3], wave=[1]) == qse.FWT_EINVAL   # 7 lane bits
    assert _split(lib, 20, 0, [13, 7], wave=[1, 1]) == 0           # column pass: 8 groups, 3 lane bits
    assert _split(lib, 20, 0, [13, 7], wave=[1, 1], gbits=[-1, 4]) == 0
    assert _split(lib, 20, 0, [13, 7], wave=[1, 1], phases=[-1, 1]) == qse.FWT_EINVAL
    # a forced group count that breaks the thread limit is rejected, not replaced
    assert _split(lib, 16, 0, [6, 10], eb=[-1, 3], gbits=[-1, 4]) == qse.FWT_EINVAL


def test_tuned_eb_zero(lib):
    # LDS tiles with row bits need at least one register bit per round.
    assert _split(lib, 12, 0, [12], eb=[0]) == qse.FWT_EINVAL
    assert _split(lib, 16, 0, [8, 8], eb=[0, 3]) == qse.FWT_EINVAL
    assert _split(lib, 16, 0, [8, 8], eb=[3, 0]) == qse.FWT_EINVAL
    assert _split(lib, 6, 1, [6], eb=[0]) == qse.FWT_EINVAL
    # the wave-tile kernel may keep every row bit in lanes
    assert _split(lib, 6, 0, [6], eb=[0], wave=[1]) == 0


FUZZ_SCRIPT = r'''
import ctypes, random, sys
sys.path.insert(0, sys.argv[1])
import quantum_state_encoding_amd as qse
lib = qse.load_library()
rng = random.Random(20240611)
counts = {}
for it in range(20000):
    n = rng.randint(1, 30)
    dtype = rng.randint(0, 1)
    npasses = rng.randint(1, 4)
    cuts = sorted(rng.sample(range(1, n), min(npasses - 1, n - 1))) if n > 1 else []
    bits = [b - a for a, b in zip([0] + cuts, cuts + [n])]
    arr = (ctypes.c_int * len(bits))(*bits)
    tun = (qse.PassTuning * len(bits))()
    for i in range(len(bits)):
        tun[i].eb = rng.randint(-1, 6)
        tun[i].gbits = rng.randint(-1, 5)
        tun[i].phases = rng.randint(-1, 3)
        tun[i].pipe = rng.randint(-1, 2)
        tun[i].wave = rng.randint(-1, 2)
    h = ctypes.c_void_p()
    st = lib.fwt_plan_create_tuned(ctypes.byref(h), n, dtype, len(bits), arr, tun)
    counts[st] = counts.get(st, 0) + 1
    if st == 0:
        npass = ctypes.c_int()
        assert lib.fwt_plan_num_passes(h, ctypes.byref(npass)) == 0 and npass.value == len(bits)
        lib.fwt_plan_destroy(h)
print(sorted(counts.items()))
'''


def test_tuned_fuzz_never_crashes():
    # Random tunings, splits, n and dtype, in a child process so that a
    # crash in plan creation fails this test instead of ending the run.
    import subprocess
    import sys
    r = subprocess.run([sys.executable, "-c", FUZZ_SCRIPT, ROOT], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, (r.returncode, r.stderr[-2000:])
    counts = dict(eval(r.stdout.strip().splitlines()[-1]))
    assert counts.get(0, 0) > 100                     # many valid plans were built
    assert set(counts) <= {0, qse.FWT_EINVAL, qse.FWT_EUNSUPPORTED}


def test_every_gpu_test_plan_is_valid(lib):
    """Each plan the GPU parity suite builds is accepted by the planner and
    has the forced properties (caught here, on the CPU)."""
    from plan_cases import (FORCED_SPLITS, LDS_SINGLE_CASES, LX_CASES, LX_COLUMN_CASES,
                            LX_PHASE_CASES, PIPE_CASES, VARIANTS, WAVE_CASES)
    for dtype, n in LDS_SINGLE_CASES:
        assert qse.Plan(n, dtype, split=(n,), wave=(0,)).pass_config(0)["wave"] == 0
    for dtype, n, split in FORCED_SPLITS:
        assert qse.Plan(n, dtype, split=split).pass_bits == list(split)
    for dtype, n, split, eb, gbits, phases in VARIANTS:
        qse.Plan(n, dtype, split=split, eb=eb, gbits=gbits, phases=phases)
    for dtype, n, split, eb, gbits, wave, batch in WAVE_CASES:
        p = qse.Plan(n, dtype, split=split, eb=eb, gbits=gbits, wave=wave)
        assert [p.pass_config(i)["wave"] for i in range(p.num_passes)] == list(wave)
    for dtype, n, split, eb, pipe, batch in PIPE_CASES:
        p = qse.Plan(n, dtype, split=split, eb=eb, pipe=pipe)
        for i, pv in enumerate(pipe):
            if pv >= 0:
                assert p.pass_config(i)["pipe"] == pv
    for dtype, n, split, eb, wave, batch in LX_CASES:
        p = qse.Plan(n, dtype, split=split, eb=eb, wave=wave)
        assert [p.pass_config(i)["wave"] for i in range(p.num_passes)] == list(wave)
    assert len(LX_CASES) == 38   # all 28 compiled variants appear
    for dtype, n, split, eb, batch in LX_PHASE_CASES:
        p = qse.Plan(n, dtype, split=split, eb=eb, phases=(1,) + (-1,) * (len(split) - 1),
                     wave=(2,) + (-1,) * (len(split) - 1))
        assert (p.pass_config(0)["wave"], p.pass_config(0)["phase_bits"]) == (2, 1)
    assert len(LX_PHASE_CASES) == 14   # all 12 compiled phased variants appear
    for dtype, n, split, eb, gbits, phases, batch in LX_COLUMN_CASES:
        k = len(split)
        knobs = {name: tuple(v if i == 1 else -1 for i in range(k))
                 for name, v in (("eb", eb), ("gbits", gbits), ("phases", phases), ("wave", 2))}
        c = qse.Plan(n, dtype, split=split, **knobs).pass_config(1)
        assert c["wave"] == 2 and c["kind"] == "column"
    assert len(LX_COLUMN_CASES) == 85  # all 78 compiled column variants appear


def test_cache_resident_tiling_of_12_bit_one_pass_plans(lib):
    """Default one-pass plans of 12 vector bits (fp32 n = 14, fp64 n = 13)
    launch eb = 3 (512 threads, one exchange) on states up to 256 MiB and
    eb = 2 (1024 threads, two exchanges) above; forced tilings, other n and
    multi-pass plans launch one tiling at every size."""
    for dtype, n, esize in (("f32", 14, 4), ("f64", 13, 8)):
        for plan in (qse.Plan(n, dtype), qse.Plan(n, dtype, split=(n,)),
                     qse.Plan(n, dtype, split=(n,), eb=(-1,))):
            assert plan.pass_config(0)["eb"] == 2
            limit = (256 << 20) // ((1 << n) * esize)      # vectors of one component
            for batch, with_im, eb in ((0, True, 3), (1, True, 3), (64, True, 3),
                                       (limit // 2, True, 3), (limit // 2 + 1, True, 2),
                                       (limit, False, 3), (limit + 1, False, 2)):
                c = plan.pass_config(0, batch, with_im)
                assert (c["eb"], c["wave"], c["block"]) == (eb, 2, 512 if eb == 3 else 1024), \
                    (dtype, batch, with_im)
            assert plan.kernel_name(0, 64) == "lx_kernel<%s, 12, 3, 3, 0, 0, true>" % (
                "float" if dtype == "f32" else "double")
        forced = qse.Plan(n, dtype, split=(n,), eb=(2,), wave=(2,))
        assert forced.pass_config(0, 64)["eb"] == 2
    for dtype, n in (("f32", 13), ("f32", 15), ("f64", 14), ("f32", 20), ("f64", 24)):
        plan = qse.Plan(n, dtype)
        for i in range(plan.num_passes):
            assert plan.pass_config(i, 1) == plan.pass_config(i)
    plan = qse.Plan(14, "f32")
    out = (ctypes.c_int * 12)()
    assert lib.fwt_plan_call_pass_config(plan._h, 0, -1, 1, out) == qse.FWT_EINVAL
    assert lib.fwt_plan_call_pass_config(plan._h, 1, 1, 1, out) == qse.FWT_EINVAL
    assert lib.fwt_plan_call_pass_config(None, 0, 1, 1, out) == qse.FWT_EINVAL
    assert lib.fwt_plan_call_pass_config(plan._h, 0, 1, 1, None) == qse.FWT_EINVAL


def test_random_plan_cases_keep_their_mix(lib):
    """The seeded random plans of the GPU suite: 80 accepted plans, each
    kernel family forced in at least 10 passes, at least 30 multi-pass
    plans, and every forced family actually selected by the planner."""
    from collections import Counter
    from plan_cases import random_plan_cases

    def accepts(dtype, n, split, kw):
        try:
            qse.Plan(n, dtype, split=split, **kw)
            return True
        except qse.FwtError:
            return False
    cases = random_plan_cases(accepts)
    assert len(cases) == 80
    modes = Counter(m for c in cases for m in c[5])
    assert all(modes[m] >= 10 for m in ("default", "lds", "wave", "lx")), modes
    assert sum(len(c[2]) > 1 for c in cases) >= 30
    for dtype, n, split, kw, batch, mode in cases:
        p = qse.Plan(n, dtype, split=split, **kw)
        for i, m in enumerate(mode):
            if m != "default" and not (dtype == "f32" and n == 1):
                assert p.pass_config(i)["wave"] == {"lds": 0, "wave": 1, "lx": 2}[m]


def test_lane_exchange_plans(lib):
    # lanes hold 6 row bits, w wave bits (default: the most threads with
    # eb >= 2), one tile per workgroup
    for dtype, vb in (("f32", 2), ("f64", 1)):
        for kr in range(8, 14):
            p = qse.Plan(kr + vb, dtype, split=(kr + vb,), wave=(2,))
            c = p.pass_config(0)
            w = kr - 6 - c["eb"]
            assert w == (min(4, kr - 8) if kr >= 10 else 1)
            assert c["block"] == 64 << w and c["lds"] == 16 << kr and c["tpw_bits"] == 0
            assert p.kernel_name(0) == "lx_kernel<%s, %d, %d, %d, 0, 0, true>" % (
                "float" if dtype == "f32" else "double", kr, c["eb"], w)
        kr = 10
        n = kr + vb
        assert _split(lib, n, vb == 1, [n], eb=[4], wave=[2]) == qse.FWT_EINVAL    # w = 0
        assert _split(lib, n, vb == 1, [n], eb=[1], wave=[2]) == qse.FWT_EINVAL    # 3 exchanges
        assert _split(lib, n + 1, vb == 1, [n + 1], eb=[2], wave=[2]) == 0       # w = 3, 2 exchanges
        assert _split(lib, n + 2, vb == 1, [n + 2], eb=[2], wave=[2]) == 0       # w = 4
        assert _split(lib, n + 3, vb == 1, [n + 3], eb=[2], wave=[2]) == qse.FWT_EINVAL  # w = 5
        assert _split(lib, n, vb == 1, [n], gbits=[1], wave=[2]) == qse.FWT_EINVAL
        assert _split(lib, n + 7, vb == 1, [n, 7], wave=[0, 2]) == 0   # column pass, 16 groups
        assert _split(lib, n + 7, vb == 1, [n, 7], gbits=[-1, 2], wave=[0, 2]) == qse.FWT_EINVAL
    assert _split(lib, 9, 0, [9], wave=[2]) == qse.FWT_EINVAL     # 7 row bits: no wave bit
    # two exchange phases: one exchange with w < eb, half the LDS
    p = qse.Plan(24, "f64", split=(14, 10), eb=(4, -1), phases=(1, -1), wave=(2, -1))
    c = p.pass_config(0)
    assert (c["wave"], c["phase_bits"], c["lds"], c["block"]) == (2, 1, 64 << 10, 512)
    assert p.kernel_name(0) == "lx_kernel<double, 13, 4, 3, 1, 0, true>"
    assert _split(lib, 15, 0, [15], eb=[3], phases=[1], wave=[2]) == qse.FWT_EINVAL  # w = eb
    assert _split(lib, 15, 0, [15], eb=[4], phases=[2], wave=[2]) == qse.FWT_EINVAL
    assert _split(lib, 12, 0, [12], eb=[3], phases=[1], wave=[2]) == qse.FWT_EUNSUPPORTED  # kr 10


def test_default_kernel_choice(lib):
    """One-pass plans of 3 <= n <= 10 default to the wave-tile kernel; other
    row passes of 8..13 vector bits to the lane-exchange kernel (except a
    multi-pass row pass of 11), and so do column passes of 8..11 bits with
    rows of at least 8 groups and of 7 bits with rows of at least 16 groups;
    the rest, and entries with any field forced, use the LDS tiles."""
    for dtype, vb in (("f32", 2), ("f64", 1)):
        for n in range(2, 15 if dtype == "f32" else 14):
            want = 1 if 3 <= n <= 10 else (2 if n - vb >= 8 else 0)
            assert qse.Plan(n, dtype).pass_config(0)["wave"] == want, (dtype, n)
            assert qse.Plan(n, dtype, split=(n,)).pass_config(0)["wave"] == want, (dtype, n)
        assert qse.Plan(8, dtype, split=(8,), eb=(3,)).pass_config(0)["wave"] == 0
        assert qse.Plan(12, dtype, split=(12,), eb=(3,)).pass_config(0)["wave"] == 0
        for split in ((5, 5), (7, 7), (2, 8), (3, 3, 4), (11, 9), (6, 10), (10, 7),
                      (10, 11), (4, 11), (5, 11)):
            p = qse.Plan(sum(split), dtype, split=split)
            lo, want = 0, []
            for i, b in enumerate(split):
                if i == 0:
                    want.append(2 if b - vb >= 8 and b - vb != 11 else 0)
                else:
                    want.append(2 if (8 <= b <= 11 and lo - vb >= 3) or (b == 7 and lo - vb >= 4)
                                else 0)
                lo += b
            assert [p.pass_config(i)["wave"] for i in range(p.num_passes)] == want, split
    for (dtype, n), (bits, wave) in {
            ("f32", 16): ([10, 6], [2, 0]), ("f32", 19): ([10, 9], [2, 2]),
            ("f32", 20): ([12, 8], [2, 2]), ("f32", 22): ([13, 9], [0, 2]),
            ("f32", 26): ([15, 11], [2, 2]), ("f64", 15): ([9, 6], [2, 0]),
            ("f64", 25): ([14, 11], [2, 2]),
            ("f64", 19): ([11, 8], [2, 2]), ("f64", 21): ([12, 9], [0, 2]),
            ("f64", 24): ([14, 10], [2, 2])}.items():
        p = qse.Plan(n, dtype)
        assert p.pass_bits == bits, (dtype, n)
        assert [p.pass_config(i)["wave"] for i in range(2)] == wave, (dtype, n)
    # 7 column bits: 16 groups, eb = 2 (the configured n = 14 split 7|7)
    assert qse.Plan(14, "f32", split=(7, 7)).kernel_name(1) == "lx_kernel<float, 7, 2, 3, 0, 4, false>"
    assert qse.Plan(17, "f32").kernel_name(1) == "lx_kernel<float, 7, 2, 3, 0, 4, false>"
    # column passes: eb = 4, two exchange phases, 16 groups up to 9 bits
    assert qse.Plan(20, "f32").kernel_name(1) == "lx_kernel<float, 8, 4, 2, 1, 4, false>"
    assert qse.Plan(24, "f64").kernel_name(1) == "lx_kernel<double, 10, 4, 3, 1, 3, false>"
    assert qse.Plan(25, "f32").kernel_name(1) == "lx_kernel<float, 10, 4, 3, 1, 3, false>"
    # 11 column bits: 8 groups, eb = 5, W = 3, two phases
    assert qse.Plan(26, "f32").kernel_name(1) == "lx_kernel<float, 11, 5, 3, 1, 3, false>"
    assert qse.Plan(25, "f64").kernel_name(1) == "lx_kernel<double, 11, 5, 3, 1, 3, false>"
    # a 13-vector-bit row pass of a two-pass plan: one exchange in two phases
    for n in (23, 24, 25):
        assert qse.Plan(n, "f64").kernel_name(0) == "lx_kernel<double, 13, 4, 3, 1, 0, true>"
    for n in (24, 25, 26):
        assert qse.Plan(n, "f32").kernel_name(0) == "lx_kernel<float, 13, 4, 3, 1, 0, true>"
    assert qse.Plan(14, "f64").kernel_name(0) == "lx_kernel<double, 13, 3, 4, 0, 0, true>"
    assert qse.Plan(15, "f32").kernel_name(0) == "lx_kernel<float, 13, 3, 4, 0, 0, true>"


def test_mfma_path_plans(lib):
    """FWT_PATH_MFMA_ABLATION: AUTO's split, with the row pass on the
    matrix-core kernel."""
    for dtype, n, bits in (("f32", 8, [8]), ("f32", 12, [12]), ("f32", 15, [15]), ("f64", 14, [14]),
                           ("f32", 20, [12, 8]), ("f64", 24, [14, 10]), ("f32", 26, [15, 11]),
                           ("f32", 27, [10, 9, 8]), ("f64", 29, [10, 10, 9])):
        p = qse.Plan(n, dtype, path=qse.PATH_MFMA_ABLATION)
        assert p.pass_bits == bits, (dtype, n)
        assert p.pass_config(0)["kind"] == "mfma"
        assert p.kernel_name(0) == "mfma_row_kernel<%s, %d>" % (
            "float" if dtype == "f32" else "double", bits[0])
        assert all(p.pass_config(i)["kind"] == "column" for i in range(1, p.num_passes))


def test_destroy(lib):
    assert lib.fwt_plan_destroy(None) == 0
    st, h = _create(lib, 8)
    assert st == 0
    assert lib.fwt_plan_destroy(h) == 0


FAKE = 0x7F0000000000  # never dereferenced: every case fails before any HIP call


@pytest.fixture
def plan10(lib):
    p = qse.Plan(10, "f32")
    yield p
    p.close()


def test_execute_rejects_before_any_hip_call(lib, plan10):
    N = 1 << 10
    ex = lambda *a: lib.fwt_execute(*a)
    h = plan10.handle
    assert ex(None, 1, 10, FAKE, FAKE + 4 * N, 1, None) == qse.FWT_EINVAL
    assert ex(h, 1, 10, None, FAKE, 1, None) == qse.FWT_EINVAL
    assert ex(h, -1, 10, FAKE, FAKE + 4 * N, 1, None) == qse.FWT_EINVAL
    assert ex(h, 1, 11, FAKE, FAKE + 8 * N, 1, None) == qse.FWT_EINVAL
    assert ex(h, 1, 10, FAKE + 4, FAKE + 4 * N, 1, None) == qse.FWT_EALIGN
    assert ex(h, 1, 10, FAKE, FAKE + 4 * N + 8, 1, None) == qse.FWT_EALIGN
    assert ex(h, 1, 10, FAKE, FAKE, 1, None) == qse.FWT_EINVAL
    assert ex(h, 2, 10, FAKE, FAKE + 4 * N, 1, None) == qse.FWT_EINVAL   # overlap
    assert ex(h, 2, 10, FAKE + 4 * N, FAKE, 1, None) == qse.FWT_EINVAL   # overlap
    assert ex(h, 1 << 62, 10, FAKE, FAKE + 16, 1, None) == qse.FWT_EINVAL  # size overflow
    # batch 0 is a no-op that touches nothing
    assert ex(h, 0, 10, FAKE, FAKE + 16, 1, None) == qse.FWT_OK
    assert lib.fwt_execute_check(h, 1, 10, FAKE + 4, None) == qse.FWT_EALIGN


def test_n0_plan_is_a_noop(lib):
    p = qse.Plan(0, "f64")
    assert p.num_passes == 0
    assert lib.fwt_execute(p.handle, 5, 0, FAKE, FAKE + 64, 1, None) == qse.FWT_OK


def test_stream_copy_rejects_before_any_hip_call(lib):
    assert lib.fwt_stream_copy(FAKE, FAKE + 4096, 100, None) == qse.FWT_EINVAL   # not x16
    assert lib.fwt_stream_copy(FAKE + 8, FAKE + 4096, 64, None) == qse.FWT_EALIGN
    assert lib.fwt_stream_copy(FAKE, FAKE + 32, 64, None) == qse.FWT_EINVAL      # overlap
    assert lib.fwt_stream_copy(None, FAKE, 64, None) == qse.FWT_EINVAL
    assert lib.fwt_stream_copy(FAKE, FAKE + 4096, 0, None) == qse.FWT_OK


def test_binding_validates_tensors_before_the_library(lib):
    """Every tensor entry point of the binding rejects a wrong dtype, a
    non-contiguous view, a size that is not whole vectors, mismatched re/im
    sizes and host tensors with ValueError, before any library call."""
    torch = pytest.importorskip("torch")
    p32, p64 = qse.Plan(4, "f32"), qse.Plan(4, "f64")
    z = torch.zeros
    bad = [(p32, z(16, dtype=torch.float64), None, "float32"),
           (p64, z(16), None, "float64"),
           (p32, z(16), z(16, dtype=torch.float64), "float32"),
           (p32, z(32)[::2], None, "contiguous"),
           (p32, z(15), None, "multiple"),
           (p32, z(16), z(32), "same number"),
           (p32, z(16), None, "device"),
           (p32, None, None, "required")]
    ev = None
    for plan, re, im, msg in bad:
        calls = [lambda: plan.execute(re, im), lambda: plan.bind(re, im),
                 lambda: plan.execute_pass(0, re, im)]
        if ev is not None:
            calls.append(lambda: plan.execute_pass_timed(0, re, im, ev, ev))
        # the ablation entry takes its dtype from re
        if re is not None and re.dtype == (torch.float32 if plan.dtype == "f32" else torch.float64):
            calls.append(lambda: qse.ablation_execute(qse.ABLATION_STAGEWISE, re, im, n=4))
        for call in calls:
            with pytest.raises(ValueError, match=msg):
                call()


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import importlib
    monkeypatch.setattr(qse, "_lib", None)
    monkeypatch.setattr(qse, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        qse.Plan(4, "f32")
    importlib.reload(qse)


def test_ablation_workspace_and_validation(lib):
    assert qse.ablation_workspace(qse.ABLATION_POPC_GEMM, 64, 14, "f32", True) == 2 * 64 * 4 << 14
    assert qse.ablation_workspace(qse.ABLATION_POPC_GEMM, 3, 10, "f64", False) == 3 * 8 << 10
    assert qse.ablation_workspace(qse.ABLATION_STAGEWISE, 64, 14, "f32", True) == 0
    ex = lib.fwt_ablation_execute
    N = 1 << 10
    # every case below fails before any HIP call
    assert ex(9, 1, 10, 0, FAKE, FAKE + 4 * N, 1, None, 0, None) == qse.FWT_EINVAL
    assert ex(qse.ABLATION_MFMA, 1, 7, 0, FAKE, FAKE + 4 * N, 1, None, 0, None) == qse.FWT_EUNSUPPORTED
    assert ex(qse.ABLATION_MFMA, 1, 30, 1, FAKE, FAKE + (8 << 30), 1, None, 0, None) == qse.FWT_EUNSUPPORTED
    assert ex(qse.ABLATION_MFMA, 1, 31, 0, FAKE, FAKE + 4 * N, 1, None, 0, None) == qse.FWT_EINVAL
    assert ex(qse.ABLATION_MFMA, 1, 10, 0, FAKE + 4, FAKE + 4 * N, 1, None, 0, None) == qse.FWT_EALIGN
    assert ex(qse.ABLATION_MFMA, 0, 10, 0, FAKE, FAKE + 4 * N, 1, None, 0, None) == qse.FWT_OK
    assert qse.ablation_workspace(qse.ABLATION_MFMA, 64, 14, "f32", True) == 0
    mt = qse.ABLATION_MFMA_TRANSPOSE
    assert qse.ablation_workspace(mt, 4, 20, "f32", True) == 2 * 4 * 4 << 20
    assert qse.ablation_workspace(mt, 4, 20, "f64", False) == 4 * 8 << 20
    for n, dtype, want in ((15, "f32", qse.FWT_EUNSUPPORTED), (31, "f32", qse.FWT_EINVAL),
                           (29, "f64", qse.FWT_EUNSUPPORTED), (16, "f32", qse.FWT_EINVAL)):
        # n = 16 passes the range check and then fails on the missing workspace
        st = lib.fwt_ablation_execute(mt, 1, n, 0 if dtype == "f32" else 1, FAKE, FAKE + (8 << 30),
                                      1, None, 0, None)
        assert st == want, (n, dtype, st)
    # INT8 / CRT: fp64, 5 <= n <= 28, residues (m = 8 moduli at n = 10, two
    # 4-byte words per element) plus per-vector scales
    oz = qse.ABLATION_OZAKI
    assert qse.ablation_workspace(oz, 4, 10, "f64", True) >= 2 * 8 * 4 * N
    assert qse.ablation_workspace(oz, 4, 10, "f64", False) < qse.ablation_workspace(oz, 4, 10, "f64", True)
    assert qse.ablation_workspace(oz, 4, 4, "f64", True) == 0
    wsb = qse.ablation_workspace(oz, 1, 10, "f64", True)
    assert ex(oz, 1, 10, 0, FAKE, FAKE + 4 * N, 1, FAKE + 16 * N, wsb, None) == qse.FWT_EUNSUPPORTED
    assert ex(oz, 1, 4, 1, FAKE, FAKE + 8 * N, 1, FAKE + 16 * N, wsb, None) == qse.FWT_EUNSUPPORTED
    assert ex(oz, 1, 29, 1, FAKE, FAKE + (8 << 29), 1, None, 0, None) == qse.FWT_EUNSUPPORTED
    assert ex(oz, 1, 10, 1, FAKE, FAKE + 8 * N, 1, None, 0, None) == qse.FWT_EINVAL
    assert ex(oz, 1, 10, 1, FAKE, FAKE + 8 * N, 1, FAKE + 16 * N, wsb - 1, None) == qse.FWT_EINVAL
    assert ex(oz, 1, 10, 1, FAKE, FAKE + 8 * N, 1, FAKE + 8, wsb, None) == qse.FWT_EALIGN
    assert ex(qse.ABLATION_STAGEWISE, 1, 1, 0, FAKE, FAKE + 64, 1, None, 0, None) == qse.FWT_EUNSUPPORTED
    assert ex(qse.ABLATION_POPC_GEMM, 1, 27, 0, FAKE, FAKE + (4 << 27), 1, None, 0, None) == qse.FWT_EUNSUPPORTED
    assert ex(qse.ABLATION_STAGEWISE, 1, 10, 0, FAKE + 4, FAKE + 4 * N, 1, None, 0, None) == qse.FWT_EALIGN
    assert ex(qse.ABLATION_STAGEWISE, 2, 10, 0, FAKE, FAKE + 4 * N, 1, None, 0, None) == qse.FWT_EINVAL
    ws = FAKE + (1 << 30)
    assert ex(qse.ABLATION_POPC_GEMM, 1, 10, 0, FAKE, FAKE + 4 * N, 1, None, 0, None) == qse.FWT_EINVAL
    assert ex(qse.ABLATION_POPC_GEMM, 1, 10, 0, FAKE, FAKE + 4 * N, 1, ws, 4 * N, None) == qse.FWT_EINVAL
    assert ex(qse.ABLATION_POPC_GEMM, 1, 10, 0, FAKE, FAKE + 4 * N, 1, FAKE + 8, 8 * N, None) == qse.FWT_EALIGN
    assert ex(qse.ABLATION_POPC_GEMM, 1, 10, 0, FAKE, FAKE + 4 * N, 1, FAKE, 8 * N, None) == qse.FWT_EINVAL
    assert ex(qse.ABLATION_STAGEWISE, 0, 10, 0, FAKE, FAKE + 4 * N, 1, None, 0, None) == qse.FWT_OK


def test_static_ablation_validation_before_any_hip_call(lib):
    """fwt_ablation_execute_static checks its size limit and every argument
    before any HIP call (there is no device here)."""
    ex = lib.fwt_ablation_execute_static
    N = 1 << 16
    big = 1 + qse.STATIC_SCRATCH_BYTES // (2 * 4 * N)
    pg, oz, mt = qse.ABLATION_POPC_GEMM, qse.ABLATION_OZAKI, qse.ABLATION_MFMA_TRANSPOSE
    assert qse.ablation_workspace(pg, big, 16, "f32", True) > qse.STATIC_SCRATCH_BYTES
    assert qse.ablation_workspace(pg, big - 1, 16, "f32", True) <= qse.STATIC_SCRATCH_BYTES
    assert ex(pg, big, 16, 0, FAKE, FAKE + (1 << 30), 1, None) == qse.FWT_ESCRATCH
    assert ex(mt, big, 16, 0, FAKE, FAKE + (1 << 30), 1, None) == qse.FWT_ESCRATCH
    assert ex(oz, 16, 20, 1, FAKE, FAKE + (1 << 30), 1, None) == qse.FWT_ESCRATCH
    assert ex(9, 1, 10, 0, FAKE, FAKE + 4 * N, 1, None) == qse.FWT_EINVAL
    assert ex(pg, -1, 10, 0, FAKE, FAKE + 4 * N, 1, None) == qse.FWT_EINVAL
    assert ex(pg, 1, 31, 0, FAKE, FAKE + 4 * N, 1, None) == qse.FWT_EINVAL
    assert ex(pg, 1, 10, 2, FAKE, FAKE + 4 * N, 1, None) == qse.FWT_EINVAL
    assert ex(pg, 1, 10, 0, FAKE + 4, FAKE + 4 * N, 1, None) == qse.FWT_EALIGN
    assert ex(pg, 1, 10, 0, FAKE, FAKE, 1, None) == qse.FWT_EINVAL
    assert ex(pg, 1, 10, 0, None, FAKE, 1, None) == qse.FWT_EINVAL
    assert ex(oz, 1, 10, 0, FAKE, FAKE + 4 * N, 1, None) == qse.FWT_EUNSUPPORTED
    assert ex(mt, 1, 15, 0, FAKE, FAKE + 4 * N, 1, None) == qse.FWT_EUNSUPPORTED
    assert ex(pg, 0, 10, 0, FAKE, FAKE + 4 * N, 1, None) == qse.FWT_OK
    assert ex(qse.ABLATION_STAGEWISE, 0, 10, 0, FAKE, FAKE + 4 * N, 1, None) == qse.FWT_OK


def test_workspace_entry_points_reject_before_any_hip_call(lib, plan10):
    """The one-pass entry points check their arguments before touching the
    device: null plan or workspace pointers, negative batches, null events
    and the base validation of fwt_execute all fail without a GPU."""
    import ctypes
    N = 1 << 10
    out = ctypes.c_size_t(7)
    bits = ctypes.c_int(3)
    h = plan10.handle
    assert lib.fwt_workspace_size(None, 1, 1, ctypes.byref(out)) == qse.FWT_EINVAL
    assert lib.fwt_workspace_size(h, -1, 1, ctypes.byref(out)) == qse.FWT_EINVAL
    assert lib.fwt_workspace_size(h, 1, 1, None) == qse.FWT_EINVAL
    # a plan other than fp32 n = 20 never uses a workspace; no device query
    assert lib.fwt_workspace_size(h, 4, 1, ctypes.byref(out)) == qse.FWT_OK
    assert out.value == 0
    p20 = qse.Plan(20, "f32", split=(10, 10))
    assert lib.fwt_workspace_size(p20.handle, 4, 1, ctypes.byref(out)) == qse.FWT_OK
    assert out.value == 0
    for dt in ("f64",):
        p = qse.Plan(20, dt)
        assert lib.fwt_workspace_size(p.handle, 4, 1, ctypes.byref(out)) == qse.FWT_OK
        assert out.value == 0
    ws = lambda *a: lib.fwt_execute_ws(*a)
    assert ws(None, 1, 10, FAKE, FAKE + 4 * N, 1, FAKE + (1 << 20), 1 << 24, None) == qse.FWT_EINVAL
    assert ws(h, 1, 10, FAKE + 4, FAKE + 4 * N, 1, None, 0, None) == qse.FWT_EALIGN
    assert ws(h, 2, 10, FAKE, FAKE + 4 * N, 1, None, 0, None) == qse.FWT_EINVAL   # overlap
    assert ws(h, 0, 10, FAKE, FAKE + 16, 1, None, 0, None) == qse.FWT_OK          # no-op
    timed = lib.fwt_execute_ws_timed
    assert timed(h, 1, 10, FAKE, FAKE + 4 * N, 1, None, 0, None, None, None) == qse.FWT_EINVAL
    assert lib.fwt_workspace_status(None, ctypes.byref(bits)) == qse.FWT_EINVAL
    assert lib.fwt_workspace_status(FAKE, None) == qse.FWT_EINVAL
