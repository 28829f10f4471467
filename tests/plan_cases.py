"""Plan parameters of the GPU parity tests, shared with the CPU tests that
check every one of them is a valid plan (so a planner change cannot break
the GPU suite unnoticed)."""

# (dtype, n, split): explicit Kronecker splits, lowest bits first
FORCED_SPLITS = [("f32", 10, (5, 5)), ("f32", 10, (2, 8)), ("f32", 10, (8, 2)), ("f32", 10, (3, 3, 4)),
    ("f32", 10, (2, 2, 2, 4)), ("f32", 14, (7, 7)), ("f32", 14, (12, 2)), ("f32", 16, (4, 12)),
    ("f32", 18, (15, 3)), ("f32", 20, (10, 10)), ("f32", 20, (8, 12)), ("f32", 20, (10, 5, 5)),
    ("f64", 10, (1, 9)), ("f64", 10, (5, 5)), ("f64", 13, (13,)), ("f64", 14, (14,)),
    ("f64", 18, (9, 9)), ("f64", 20, (8, 12)), ("f64", 22, (10, 12)), ("f64", 21, (7, 7, 7))]


def _variants():
    out = [("f64", 14, (4, 10), (-1, 4), (-1, 3), (-1, 1)),
           ("f64", 14, (4, 10), (-1, 4), (-1, 3), (-1, 2)),
           ("f64", 15, (4, 11), (-1, 4), (-1, 3), (-1, 2)),
           ("f32", 16, (5, 11), (-1, 4), (-1, 3), (-1, 2)),
           ("f32", 16, (6, 10), (-1, 3), (-1, 3), (-1, 1)),
           ("f32", 16, (6, 10), (-1, 4), (-1, 4), (-1, 2)),
           ("f32", 21, (12, 9), (-1, 4), (-1, 4), (-1, 1))]
    for dtype in ("f32", "f64"):
        vb = 2 if dtype == "f32" else 1
        for row_eb in (3, 4, 5):
            out.append((dtype, 8 + vb + 8, (8 + vb, 8), (row_eb, 4), (-1, -1), None))
        for col_eb in (3, 4):
            for gb in range(0, 5):
                out.append((dtype, 8 + vb + 8, (8 + vb, 8), (4, col_eb), (-1, gb), None))
        out.append((dtype, 3 + vb + 10, (3 + vb, 10), (3, 4), (-1, 0), None))
        out.append((dtype, 12 + vb, (12 + vb,), (5,), (-1,), None))
        out.append((dtype, 12 + vb, (12 + vb,), (3,), (-1,), None))
    return out
VARIANTS = _variants()

# (dtype, n, split, eb, pipe, batch): the persistent pipelined kernel forced
# on (1) or off (0) per pass
PIPE_CASES = [
    ("f64", 18, (14, 4), (4, -1), (1, 0), 3), ("f64", 18, (14, 4), (4, -1), (0, 0), 3),
    ("f32", 17, (15, 2), (4, -1), (1, 0), 2), ("f32", 16, (13, 3), (4, -1), (1, 0), 5),
    ("f64", 16, (13, 3), (4, -1), (1, 0), 3), ("f64", 20, (10, 10), (-1, 4), (0, 1), 2),
    ("f32", 19, (9, 10), (-1, 4), (-1, 1), 1), ("f64", 24, (14, 10), (4, -1), (1, 0), 1),
    ("f32", 14, (14,), (4,), (1,), 7), ("f32", 20, (13, 7), (4, 3), (1, 1), 2)]

# (dtype, n, split, eb, gbits, wave, batch): the wave-tile kernel (whole
# tile in one wave; lane bits crossed with DPP, ds_swizzle and permlane
# swaps), row and column passes, every lane-bit count and column-group count
WAVE_CASES = [
    ("f32", 12, (12,), None, None, (1,), 3), ("f32", 13, (13,), None, None, (1,), 2),
    ("f32", 10, (10,), None, None, (1,), 5), ("f32", 5, (5,), None, None, (1,), 9),
    ("f32", 8, (8,), None, None, (1,), 33), ("f32", 3, (3,), None, None, (1,), 7),
    ("f64", 12, (12,), None, None, (1,), 2), ("f64", 7, (7,), None, None, (1,), 9),
    ("f64", 2, (2,), None, None, (1,), 5), ("f64", 9, (9,), None, None, (1,), 4),
    ("f32", 16, (9, 7), None, None, (1, 1), 1), ("f32", 16, (9, 7), None, (-1, 4), (1, 1), 1),
    ("f64", 15, (8, 7), None, (-1, 2), (0, 1), 1), ("f32", 14, (7, 7), None, (-1, 1), (1, 1), 2),
    ("f32", 13, (4, 9), None, (-1, 0), (1, 1), 3), ("f64", 12, (3, 9), None, (-1, 0), (1, 1), 3),
    ("f32", 20, (13, 7), None, None, (1, 1), 2), ("f32", 20, (13, 7), None, (-1, 4), (1, 1), 2),
    ("f64", 18, (11, 7), None, None, (1, 1), 2), ("f32", 12, (12,), (5,), None, (1,), 2),
    ("f32", 14, (10, 4), None, (-1, 3), (1, 1), 3)]

# (dtype, n): one-pass plans with the LDS-tile kernel forced (wave 0) where
# the default plan picks the wave-tile kernel (3 <= n <= 10), and either side
LDS_SINGLE_CASES = [(dt, n) for dt in ("f32", "f64") for n in range(2, 12)]


# (dtype, n, split, eb, wave, batch): the lane-exchange row kernel (lanes hold
# the 6 lowest row bits, LDS exchanges move the wave bits into registers),
# every compiled (row bits, eb, wave bits) variant as a one-pass plan, and
# as the row pass of two-pass plans
def _lx_cases():
    out = []
    for dtype, vb in (("f32", 2), ("f64", 1)):
        for kr in range(8, 14):
            for w in (1, 2, 3, 4):
                eb = kr - 6 - w
                if 2 <= eb <= 5 or eb == w == 1:
                    out.append((dtype, kr + vb, (kr + vb,), (eb,), (2,), 3))
    out += [("f32", 20, (13, 7), (3, -1), (2, 0), 2), ("f32", 20, (13, 7), (4, -1), (2, 0), 2),
            ("f64", 24, (14, 10), (4, -1), (2, 0), 1), ("f64", 20, (12, 8), None, (2, 0), 3),
            ("f32", 18, (11, 7), None, (2, 0), 5), ("f32", 14, (14,), None, (2,), 65),
            ("f32", 12, (12,), None, (2,), 1), ("f64", 13, (13,), None, (2,), 129),
            ("f32", 20, (13, 7), (2, -1), (2, 0), 2), ("f32", 15, (15,), (3,), (2,), 33)]
    return out
LX_CASES = _lx_cases()

# (dtype, n, split, eb, batch): the lane-exchange kernel with its single
# exchange in two phases (half the LDS), every compiled variant
def _lx_phase_cases():
    out = []
    for dtype, vb in (("f32", 2), ("f64", 1)):
        for kr in range(11, 14):
            for w in (1, 2, 3, 4):
                eb = kr - 6 - w
                if 2 <= eb <= 5 and w < eb:
                    out.append((dtype, kr + vb, (kr + vb,), (eb,), 3))
    out += [("f64", 24, (14, 10), (4, -1), 1), ("f32", 20, (13, 7), (4, -1), 2)]
    return out
LX_PHASE_CASES = _lx_phase_cases()


# (dtype, n, split, eb, gbits, phases, batch): the lane-exchange kernel on a
# column pass (lanes hold 8 or 16 column groups and 3 or 2 row bits), every
# compiled variant, with 4-8 column blocks per row and two outer indices
def _lx_column_cases():
    out = []
    for dtype, vb in (("f32", 2), ("f64", 1)):
        for gb in (3, 4):
            lr = 6 - gb
            for kr in range(6, 12):
                for w in (1, 2, 3, 4):
                    eb = kr - lr - w
                    if not (2 <= eb <= 5 or eb == w == 1):
                        continue
                    for ph in (0, 1):
                        if ph == 0 and kr + gb > 13:
                            continue
                        if ph == 1 and not (11 <= kr + gb <= 14 and w < eb):
                            continue
                        lo = gb + vb + 2          # 4 column blocks per row
                        out.append((dtype, lo + kr + 1, (lo, kr, 1), eb, gb, ph, 1))
    out += [("f32", 20, (12, 8), -1, -1, -1, 3), ("f64", 24, (14, 10), -1, -1, -1, 1),
            ("f64", 20, (11, 9), -1, -1, -1, 2), ("f32", 19, (10, 9), -1, 3, -1, 5),
            # default 11-bit columns whose rows are exactly one tile wide
            ("f32", 16, (5, 11), -1, -1, -1, 3), ("f64", 15, (4, 11), -1, -1, -1, 2),
            ("f32", 19, (8, 11), -1, -1, -1, 1)]
    return out
LX_COLUMN_CASES = _lx_column_cases()


# Seeded random plans: a Kronecker split of n into 1-4 factors and, per
# pass, the default kernel or one family forced (LDS tiles, wave tiles,
# lane exchange) with random tiling fields.  `valid(dtype, n, split, kw)`
# tells whether the planner accepts the plan; only accepted plans are kept.
# Each case: (dtype, n, split, kw, batch), kw the Plan keyword arguments.
RANDOM_MODES = ("default", "lds", "wave", "lx")


def random_plan_cases(valid, count=80, seed=20_261_202, batches=None):
    """`count` random (dtype, n, split, tuning, batch, modes) cases that
    `valid` accepts: batches of 1-5 vectors, or one of `batches` (cases
    whose state would pass 2^22 elements per component are skipped then)."""
    import numpy as np
    rng = np.random.default_rng(seed)

    def pick(choices):
        # the default (-1) half of the time, else one of choices
        return -1 if rng.random() < 0.5 else int(rng.choice(choices))

    out = []
    tries = 0
    while len(out) < count and tries < 200_000:
        tries += 1
        dtype = ("f32", "f64")[int(rng.integers(0, 2))]
        n = int(rng.integers(4, 21))
        npasses = int(rng.choice([1, 2, 3, 4], p=[0.15, 0.35, 0.3, 0.2]))
        if npasses > n:
            continue
        cuts = sorted(int(c) for c in rng.choice(np.arange(1, n), npasses - 1, replace=False))
        split = tuple(b - a for a, b in zip([0] + cuts, cuts + [n]))
        fields = {f: [] for f in ("eb", "gbits", "phases", "pipe", "wave")}
        modes = []
        for i in range(npasses):
            mode = RANDOM_MODES[int(rng.integers(0, len(RANDOM_MODES)))]
            modes.append(mode)
            v = {f: -1 for f in fields}
            if mode == "lds":
                v["wave"] = 0
                v["eb"] = pick([1, 2, 3, 4, 5])
                v["gbits"] = pick([0, 1, 2, 3, 4]) if i else -1
                v["phases"] = pick([0, 1, 2]) if i else -1
                v["pipe"] = pick([0, 1])
            elif mode == "wave":
                v["wave"] = 1
                v["eb"] = pick([0, 1, 2, 3, 4, 5])
                v["gbits"] = pick([0, 1, 2, 3, 4]) if i else -1
            elif mode == "lx":
                v["wave"] = 2
                v["eb"] = pick([1, 2, 3, 4, 5])
                v["gbits"] = pick([3, 4]) if i else -1
                v["phases"] = pick([0, 1])
            for f in fields:
                fields[f].append(v[f])
        kw = {f: tuple(vals) for f, vals in fields.items()}
        if not valid(dtype, n, split, kw):
            continue
        if batches is None:
            batch = max(1, min(int(rng.integers(1, 6)), (1 << 22) >> n))
        else:
            batch = int(rng.choice(batches))
            if batch > (1 << 22) >> n:
                continue
        out.append((dtype, n, split, kw, batch, tuple(modes)))
    return out
