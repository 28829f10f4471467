"""fwt_ablation_execute_static, the ablation entry point that allocates
nothing (its workspace is the library's static scratch array), against
fwt_ablation_execute with a caller workspace, through the C ABI.

For each kind that needs a workspace, two calls run in a row on the same
device, the second on a smaller input, so the second finds the first's
data in the scratch array.  Both must equal the caller-workspace result
bit for bit (the same kernels on the same inputs), and integer inputs must
also equal the oracle exactly.
"""
import ctypes
import sys

import numpy as np
import pytest

import oracle
import quantum_state_encoding_amd as qse

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

DT = {"f32": 0, "f64": 1}
NP = {"f32": np.float32, "f64": np.float64}


def say(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def state(batch, n, dtype, seed, ints):
    rng = np.random.default_rng(seed)
    shape = (batch, 1 << n)
    if ints:
        return (rng.integers(-8, 9, size=shape).astype(NP[dtype]),
                rng.integers(-8, 9, size=shape).astype(NP[dtype]))
    return (rng.standard_normal(shape).astype(NP[dtype]),
            rng.standard_normal(shape).astype(NP[dtype]))


def via_workspace(kind, re, im, n, dtype, normalize):
    tre = torch.from_numpy(re).cuda()
    tim = torch.from_numpy(im).cuda() if im is not None else None
    wsb = qse.ablation_workspace(kind, re.shape[0], n, dtype, im is not None)
    ws = torch.empty(max(wsb, 16) // 4, dtype=torch.float32, device="cuda")
    st = qse.load_library().fwt_ablation_execute(
        kind, re.shape[0], n, DT[dtype], ctypes.c_void_p(tre.data_ptr()),
        ctypes.c_void_p(tim.data_ptr() if tim is not None else None), int(normalize),
        ctypes.c_void_p(ws.data_ptr()), ws.numel() * 4,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == qse.FWT_OK, st
    torch.cuda.synchronize()
    return tre.cpu().numpy(), (tim.cpu().numpy() if tim is not None else None)


def via_static(kind, re, im, n, dtype, normalize):
    tre = torch.from_numpy(re).cuda()
    tim = torch.from_numpy(im).cuda() if im is not None else None
    st = qse.load_library().fwt_ablation_execute_static(
        kind, re.shape[0], n, DT[dtype], ctypes.c_void_p(tre.data_ptr()),
        ctypes.c_void_p(tim.data_ptr() if tim is not None else None), int(normalize),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == qse.FWT_OK, st
    torch.cuda.synchronize()
    return tre.cpu().numpy(), (tim.cpu().numpy() if tim is not None else None)


# (kind, dtype, n, batch of the first call, (n, batch) of the second, smaller
# call); each first call needs several MiB of the scratch array.
CASES = [
    ("popc_gemm", qse.ABLATION_POPC_GEMM, "f32", 14, 64, (12, 16)),
    ("popc_gemm", qse.ABLATION_POPC_GEMM, "f64", 12, 96, (12, 5)),
    ("ozaki", qse.ABLATION_OZAKI, "f64", 14, 16, (10, 3)),
    ("mfma_transpose", qse.ABLATION_MFMA_TRANSPOSE, "f32", 16, 24, (16, 2)),
    ("mfma_transpose", qse.ABLATION_MFMA_TRANSPOSE, "f64", 17, 8, (16, 3)),
]


@pytest.mark.parametrize("name,kind,dtype,n,batch,second", CASES,
                         ids=["%s-%s-n%d" % (c[0], c[2], c[3]) for c in CASES])
@pytest.mark.parametrize("ints", [True, False], ids=["int", "gauss"])
def test_static_scratch_matches_caller_workspace(name, kind, dtype, n, batch, second, ints):
    assert qse.ablation_workspace(kind, batch, n, dtype, True) <= qse.STATIC_SCRATCH_BYTES
    for call, (nn, bb) in enumerate(((n, batch), second)):
        say("static scratch %s %s n=%d batch=%d call %d %s" % (name, dtype, nn, bb, call,
                                                              "int" if ints else "gauss"))
        re, im = state(bb, nn, dtype, 1000 * call + nn, ints)
        normalize = nn % 2 == 0
        s_re, s_im = via_static(kind, re, im, nn, dtype, normalize)
        w_re, w_im = via_workspace(kind, re, im, nn, dtype, normalize)
        assert np.array_equal(s_re, w_re) and np.array_equal(s_im, w_im)
        if ints:
            assert np.array_equal(s_re.astype(np.float64), oracle.fwt(re, nn, normalize))
            assert np.array_equal(s_im.astype(np.float64), oracle.fwt(im, nn, normalize))


def test_static_scratch_real_only_and_limits():
    kind = qse.ABLATION_POPC_GEMM
    say("static scratch real-only popc_gemm f32 n=13")
    re, _ = state(40, 13, "f32", 7, True)
    s_re, _ = via_static(kind, re, None, 13, "f32", False)
    w_re, _ = via_workspace(kind, re, None, 13, "f32", False)
    assert np.array_equal(s_re, w_re)
    assert np.array_equal(s_re.astype(np.float64), oracle.fwt(re, 13, False))
    # Beyond the array: FWT_ESCRATCH, and the data are left as they were.
    say("static scratch beyond its size")
    big = 1 + qse.STATIC_SCRATCH_BYTES // (2 * 4 << 16)
    tre = torch.ones(big, 1 << 16, device="cuda")
    tim = torch.ones_like(tre)
    with pytest.raises(qse.FwtError) as ei:
        qse.ablation_execute_static(kind, tre, tim, n=16)
    assert ei.value.status == qse.FWT_ESCRATCH
    torch.cuda.synchronize()
    assert bool((tre == 1).all()) and bool((tim == 1).all())
    # A kind without a workspace runs as fwt_ablation_execute does.
    say("static scratch stagewise f32 n=12")
    re, im = state(8, 12, "f32", 11, True)
    s_re, s_im = via_static(qse.ABLATION_STAGEWISE, re, im, 12, "f32", True)
    assert np.array_equal(s_re.astype(np.float64), oracle.fwt(re, 12, True))
    assert np.array_equal(s_im.astype(np.float64), oracle.fwt(im, 12, True))
