"""Parity of the one-HBM-pass fp32 n = 20 kernel (fwt_execute_ws) with the
CPU oracle, through the C ABI, and its argument and workspace contract.

Bars as in test_gpu_parity: integer inputs bit-exact (every partial sum is
an integer below 2^24 and 2^-10 is a power of two), Gaussian unit-norm
inputs within 1e-5 * ||x||_2 per vector of the fp64 oracle.  After every
call the workspace's error word must be 0 (no wait ran out, every
workgroup ran on the XCD its index implies).
"""
import os
import sys

import numpy as np
import pytest

import oracle
import quantum_state_encoding_amd as qse
import workloads

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

N20 = 20


def say(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def ints(shape, seed):
    return np.random.default_rng(seed).integers(-8, 9, size=shape).astype(np.float32)


@pytest.fixture(scope="module")
def plan():
    p = qse.Plan(N20, "f32")
    if p.workspace_size(1) == 0:
        pytest.fail("the one-pass kernel is not available on this device")
    return p


def workspace(plan, batch, with_im=True):
    return torch.empty(plan.workspace_size(batch, with_im), dtype=torch.uint8, device="cuda")


def run_ws(plan, re, im, normalize, ws=None):
    tre = to_dev(re)
    tim = to_dev(im) if im is not None else None
    if ws is None:
        ws = workspace(plan, re.shape[0], im is not None)
    plan.execute_ws(tre, tim, normalize=normalize, workspace=ws)
    torch.cuda.synchronize()
    assert qse.workspace_status(ws) == 0
    return tre.cpu().numpy(), (tim.cpu().numpy() if tim is not None else None)


@pytest.mark.parametrize("batch,with_im,normalize", [(1, True, True), (1, False, False),
                                                      (2, True, False), (3, True, True),
                                                      (3, False, True), (5, True, True),
                                                      (8, True, False), (9, True, True)])
def test_integer_bit_exact(plan, batch, with_im, normalize):
    """Every element of every vector equals the oracle's transform; ragged
    component counts (1, 3, 5, 10, 18: fewer components than groups, or
    not a multiple of the 8 XCDs) included."""
    say("onepass int batch=%d im=%s normalize=%s" % (batch, with_im, normalize))
    re = ints((batch, 1 << N20), 700 + batch)
    im = ints((batch, 1 << N20), 800 + batch) if with_im else None
    gre, gim = run_ws(plan, re, im, normalize)
    assert np.array_equal(gre.astype(np.float64), oracle.fwt(re, N20, normalize))
    if with_im:
        assert np.array_equal(gim.astype(np.float64), oracle.fwt(im, N20, normalize))


def test_gaussian_within_tolerance(plan):
    say("onepass gauss batch=4")
    w = workloads.custom(N20, 4, "f32", "gauss", True, seed=20_004)
    re, im = workloads.gen(w)
    gre, gim = run_ws(plan, re, im, True)
    ore, oim = oracle.fwt_complex(re, im, N20, True)
    for b in range(4):
        nx = np.sqrt(np.sum(re[b].astype(np.float64) ** 2) + np.sum(im[b].astype(np.float64) ** 2))
        err = max(np.abs(gre[b] - ore[b]).max(), np.abs(gim[b] - oim[b]).max())
        assert err <= 1e-5 * nx, "vector %d: %.3g" % (b, err / nx)


def test_full_size_n20_b256(plan):
    """The benchmark's workload through the one-pass kernel: every vector
    against the oracle's fp64 transform (threaded form, blocks of vectors),
    and norm preservation of every vector."""
    w = workloads.WORKLOADS["n20_b256_f32"]
    say("onepass full size %s" % w.name)
    re, im = workloads.gen(w)
    tre, tim = to_dev(re), to_dev(im)
    ws = workspace(plan, w.batch)
    plan.execute_ws(tre, tim, normalize=True, workspace=ws)
    torch.cuda.synchronize()
    assert qse.workspace_status(ws) == 0
    ny = torch.sqrt((tre.double() ** 2).sum(1) + (tim.double() ** 2).sum(1)).cpu().numpy()
    nx = np.sqrt((re.astype(np.float64) ** 2).sum(1) + (im.astype(np.float64) ** 2).sum(1))
    assert np.abs(ny - nx).max() <= 1e-5 * nx.max()
    threads = min(16, len(os.sched_getaffinity(0)))
    blk = 8
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
        assert (ratio <= 1e-5).all(), "vectors %d..%d: %.3g" % (b0, b1 - 1, ratio.max())
    say("onepass full size: max|err|/||x|| = %.3g" % worst)
    del tre, tim
    torch.cuda.empty_cache()


def test_equals_two_pass_on_integers_and_repeats(plan):
    """37 vectors (74 components): the one-pass result equals fwt_execute's
    two passes bit for bit, and twenty calls on the same input give the same
    bits (the DPP stages' wait states, the ring's reuse across calls)."""
    say("onepass vs two-pass batch=37, twenty repeats")
    re = ints((37, 1 << N20), 937)
    im = ints((37, 1 << N20), 938)
    src_re, src_im = to_dev(re), to_dev(im)
    a_re, a_im = src_re.clone(), src_im.clone()
    plan.execute(a_re, a_im, normalize=True)
    ws = workspace(plan, 37)
    for rep in range(20):
        b_re, b_im = src_re.clone(), src_im.clone()
        plan.execute_ws(b_re, b_im, normalize=True, workspace=ws)
        torch.cuda.synchronize()
        assert qse.workspace_status(ws) == 0, "call %d" % rep
        assert torch.equal(a_re, b_re) and torch.equal(a_im, b_im), "call %d" % rep


def test_batch_past_the_benchmark_without_im(plan):
    """300 vectors with no imaginary plane: 300 components, 37 or 38 per
    XCD, so the groups' queues run past the benchmark's 32 components per
    group and end unevenly.  Bit-for-bit equal to fwt_execute's two passes
    on integers (|values| <= 8 * 2^20 stay exact in fp32), and sampled
    vectors equal the oracle's transform."""
    batch = 300
    say("onepass batch=%d without im" % batch)
    re = ints((batch, 1 << N20), 1300)
    src = to_dev(re)
    a = src.clone()
    plan.execute(a, None, normalize=False)
    ws = workspace(plan, batch, False)
    b = src.clone()
    plan.execute_ws(b, None, normalize=False, workspace=ws)
    torch.cuda.synchronize()
    assert qse.workspace_status(ws) == 0
    assert torch.equal(a, b)
    for i in (0, 7, 8, 151, 299):
        assert np.array_equal(b[i].cpu().numpy().astype(np.float64),
                              oracle.fwt(re[i:i + 1], N20, False)[0]), "vector %d" % i
    del src, a, b
    torch.cuda.empty_cache()


def test_successive_batches_share_one_workspace(plan):
    """Calls of different sizes in a row on one workspace (each call clears
    its header; the queue and the next-index words start over): every call
    equals fwt_execute's two passes bit for bit and leaves no error bits."""
    ws = workspace(plan, 300)
    for k, batch in enumerate((256, 1, 37, 300, 2, 256)):
        say("onepass successive batch=%d" % batch)
        re = ints((batch, 1 << N20), 2000 + k)
        im = ints((batch, 1 << N20), 3000 + k) if batch % 2 == 0 else None
        src_re = to_dev(re)
        src_im = to_dev(im) if im is not None else None
        a_re = src_re.clone()
        a_im = src_im.clone() if src_im is not None else None
        plan.execute(a_re, a_im, normalize=True)
        plan.execute_ws(src_re, src_im, normalize=True, workspace=ws)
        torch.cuda.synchronize()
        assert qse.workspace_status(ws) == 0, "batch %d" % batch
        assert torch.equal(a_re, src_re), "batch %d" % batch
        if im is not None:
            assert torch.equal(a_im, src_im), "batch %d" % batch
        del src_re, src_im, a_re, a_im
    torch.cuda.empty_cache()


def test_involution_gaussian(plan):
    """Two normalised calls give back the input within tolerance."""
    say("onepass involution")
    w = workloads.custom(N20, 6, "f32", "gauss", True, seed=20_006)
    re, im = workloads.gen(w)
    tre, tim = to_dev(re), to_dev(im)
    ws = workspace(plan, 6)
    for _ in range(2):
        plan.execute_ws(tre, tim, normalize=True, workspace=ws)
    torch.cuda.synchronize()
    assert qse.workspace_status(ws) == 0
    assert np.abs(tre.cpu().numpy() - re).max() <= 2e-5
    assert np.abs(tim.cpu().numpy() - im).max() <= 2e-5


def test_graph_capture_and_replay(plan):
    """bind_ws captured into a HIP graph (the header is cleared by a kernel,
    not a memset) and replayed three times with eager work in between:
    every replay equals the eager call bit for bit."""
    say("onepass graph")
    w = workloads.custom(N20, 3, "f32", "gauss", True, seed=20_033)
    re0, im0 = workloads.gen(w)
    ws = workspace(plan, 3)
    e_re, e_im = to_dev(re0), to_dev(im0)
    plan.execute_ws(e_re, e_im, normalize=True, workspace=ws)
    torch.cuda.synchronize()
    x_re, x_im = to_dev(re0), to_dev(im0)
    g_re, g_im = torch.empty_like(x_re), torch.empty_like(x_im)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        fn = plan.bind_ws(g_re, g_im, normalize=True, workspace=ws, stream=s)
        g_re.copy_(x_re)
        g_im.copy_(x_im)
        fn()
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
        assert qse.workspace_status(ws) == 0
        assert torch.equal(g_re, e_re) and torch.equal(g_im, e_im), "replay %d" % rep
        junk = torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")
        torch.cuda.synchronize()
        del junk


def test_timed_call_records_the_kernel(plan):
    say("onepass timed")
    re = ints((4, 1 << N20), 44)
    im = ints((4, 1 << N20), 45)
    tre, tim = to_dev(re), to_dev(im)
    ws = workspace(plan, 4)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    plan.execute_ws_timed(tre, tim, ws, start, stop, normalize=False)
    torch.cuda.synchronize()
    assert qse.workspace_status(ws) == 0
    assert 0.0 < start.elapsed_time(stop) < 1000.0
    assert np.array_equal(tre.cpu().numpy().astype(np.float64), oracle.fwt(re, N20, False))


def test_workspace_contract(plan):
    """Missing, small, misaligned or overlapping workspaces are rejected
    before anything runs; other plans ignore the workspace and run
    fwt_execute's passes."""
    say("onepass workspace contract")
    re = to_dev(ints((2, 1 << N20), 1))
    im = to_dev(ints((2, 1 << N20), 2))
    need = plan.workspace_size(2)
    assert need >= 16 << 20
    assert plan.workspace_size(2, with_im=False) == need
    assert plan.workspace_size(0) == 0
    big = torch.empty(need + 512, dtype=torch.uint8, device="cuda")
    for bad, status in ((None, qse.FWT_EINVAL), (big[:need - 16], qse.FWT_EINVAL),
                        (big[16:need + 16], qse.FWT_EALIGN)):
        with pytest.raises(qse.FwtError) as e:
            plan.execute_ws(re, im, workspace=bad)
        assert e.value.status == status
    # a workspace inside the state
    state = torch.zeros(8 << 20, dtype=torch.float32, device="cuda")
    with pytest.raises(qse.FwtError) as e:   # large enough, aligned, but over re's last 4 KiB
        plan.execute_ws(state[: 1 << 20].view(1, -1), None,
                        workspace=state[(1 << 20) - 1024:].view(torch.uint8))
    assert e.value.status == qse.FWT_EINVAL
    # the untouched inputs still transform correctly afterwards
    ref_re, ref_im = re.clone(), im.clone()
    plan.execute(ref_re, ref_im, normalize=True)
    plan.execute_ws(re, im, normalize=True, workspace=big[:need])
    torch.cuda.synchronize()
    assert torch.equal(re, ref_re) and torch.equal(im, ref_im)
    # other plans: size 0, workspace ignored (None accepted)
    for p, n in ((qse.Plan(20, "f32", split=(10, 10)), 20), (qse.Plan(19, "f32"), 19),
                 (qse.Plan(20, "f64"), 20)):
        assert p.workspace_size(4) == 0
        dt = torch.float64 if p.dtype == "f64" else torch.float32
        a = torch.randint(-8, 9, (2, 1 << n), device="cuda").to(dt)
        b = a.clone()
        p.execute(a, None, normalize=False)
        p.execute_ws(b, None, normalize=False, workspace=None)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
