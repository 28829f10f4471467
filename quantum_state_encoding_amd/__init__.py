"""Batched in-place Walsh-Hadamard transform on MI355X (gfx950).

A thin ctypes binding over ``libfwt.so`` (the C ABI declared in
``include/fwt.h``).  This module only marshals arguments: every step of the
transform runs in the library's HIP kernels.  PyTorch is used for device
memory and streams only.  If the library has not been built the import
still succeeds, but every call raises: there is no fallback.

Example::

    import torch, quantum_state_encoding_amd as qse
    re = torch.randn(64, 4096, device="cuda"); im = torch.randn_like(re)
    plan = qse.Plan(12, "f32")
    plan.execute(re, im, normalize=True)   # in place, on the current stream
"""
import ctypes
import os

__all__ = ["Plan", "FwtError", "execute", "stream_copy", "library_path", "load_library",
           "ablation_workspace", "ablation_execute", "ABLATION_STAGEWISE", "ABLATION_POPC_GEMM",
           "ABLATION_MFMA", "ABLATION_OZAKI", "ABLATION_MFMA_TRANSPOSE", "PassTuning",
           "PATH_AUTO", "PATH_SINGLE_BLOCK", "PATH_MULTIPASS", "PATH_MFMA_ABLATION",
           "FWT_OK", "FWT_EINVAL", "FWT_EALIGN", "FWT_EUNSUPPORTED", "FWT_EHIP",
           "FWT_ENOMEM", "FWT_ESCRATCH", "STATIC_SCRATCH_BYTES", "ablation_execute_static",
           "EXPORTED_SYMBOLS", "workspace_status"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfwt.so")

FWT_OK, FWT_EINVAL, FWT_EALIGN, FWT_EUNSUPPORTED, FWT_EHIP, FWT_ENOMEM = 0, -1, -2, -3, -4, -5
FWT_ESCRATCH = -6
STATIC_SCRATCH_BYTES = 32 << 20   # FWT_STATIC_SCRATCH_BYTES
PATH_AUTO, PATH_SINGLE_BLOCK, PATH_MULTIPASS, PATH_MFMA_ABLATION = 0, 1, 2, 3
_DTYPES = {"f32": 0, "f64": 1}

# Every symbol include/fwt.h declares.
EXPORTED_SYMBOLS = ("fwt_plan_create", "fwt_plan_create_split", "fwt_plan_create_tuned",
                    "fwt_execute", "fwt_execute_pass", "fwt_execute_pass_timed",
                    "fwt_execute_check", "fwt_workspace_size", "fwt_execute_ws",
                    "fwt_execute_ws_timed", "fwt_workspace_status",
                    "fwt_plan_num_passes", "fwt_plan_pass_config", "fwt_plan_call_pass_config",
                    "fwt_plan_pass_bits",
                    "fwt_plan_destroy", "fwt_strerror", "fwt_last_hip_error",
                    "fwt_stream_copy", "fwt_plan_chunk_vectors", "fwt_plan_call_schedule",
                    "fwt_ablation_workspace",
                    "fwt_ablation_execute", "fwt_ablation_execute_static")

_lib = None


class PassTuning(ctypes.Structure):
    """fwt_pass_tuning: per-pass tiling overrides (-1 = default)."""
    _fields_ = [("eb", ctypes.c_int), ("gbits", ctypes.c_int), ("phases", ctypes.c_int),
                ("pipe", ctypes.c_int), ("wave", ctypes.c_int)]


class FwtError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, status, what):
        self.status = status
        msg = "%s failed: %s (status %d)" % (what, _strerror(status), status)
        if status == FWT_EHIP:
            msg += ", HIP error %d" % load_library().fwt_last_hip_error()
        super().__init__(msg)


def library_path():
    return _LIB_PATH


def load_library():
    """Load libfwt.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libfwt.so not found at %s: build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'` or "
                          "`python quantum_state_encoding_amd/build.py`" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    pi = ctypes.POINTER(ctypes.c_int)
    lib.fwt_plan_create.argtypes = [ctypes.POINTER(vp), i32, i32, i32]
    lib.fwt_plan_create_split.argtypes = [ctypes.POINTER(vp), i32, i32, i32, pi]
    lib.fwt_plan_create_tuned.argtypes = [ctypes.POINTER(vp), i32, i32, i32, pi,
                                          ctypes.POINTER(PassTuning)]
    lib.fwt_plan_chunk_vectors.argtypes = [vp, i64, i32, ctypes.POINTER(i64)]
    lib.fwt_plan_call_schedule.argtypes = [vp, i64, i32, pi, pi, ctypes.POINTER(i64)]
    lib.fwt_plan_call_schedule.restype = i32
    lib.fwt_execute.argtypes = [vp, i64, i32, vp, vp, i32, vp]
    lib.fwt_execute_pass.argtypes = [vp, i32, i64, i32, vp, vp, i32, vp]
    lib.fwt_execute_pass_timed.argtypes = [vp, i32, i64, i32, vp, vp, i32, vp, vp, vp]
    lib.fwt_execute_check.argtypes = [vp, i64, i32, vp, vp]
    lib.fwt_plan_num_passes.argtypes = [vp, pi]
    lib.fwt_plan_pass_bits.argtypes = [vp, i32, pi]
    lib.fwt_plan_pass_config.argtypes = [vp, i32, pi]
    lib.fwt_plan_call_pass_config.argtypes = [vp, i32, i64, i32, pi]
    lib.fwt_plan_destroy.argtypes = [vp]
    lib.fwt_strerror.argtypes = [i32]
    lib.fwt_strerror.restype = ctypes.c_char_p
    lib.fwt_last_hip_error.argtypes = []
    lib.fwt_stream_copy.argtypes = [vp, vp, i64, vp]
    lib.fwt_ablation_workspace.argtypes = [i32, i64, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.fwt_ablation_execute.argtypes = [i32, i64, i32, i32, vp, vp, i32, vp, ctypes.c_size_t, vp]
    lib.fwt_ablation_execute_static.argtypes = [i32, i64, i32, i32, vp, vp, i32, vp]
    lib.fwt_workspace_size.argtypes = [vp, i64, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.fwt_execute_ws.argtypes = [vp, i64, i32, vp, vp, i32, vp, ctypes.c_size_t, vp]
    lib.fwt_execute_ws_timed.argtypes = [vp, i64, i32, vp, vp, i32, vp, ctypes.c_size_t, vp,
                                         vp, vp]
    lib.fwt_workspace_status.argtypes = [vp, pi]
    for name in ("fwt_workspace_size", "fwt_execute_ws", "fwt_execute_ws_timed",
                 "fwt_workspace_status", "fwt_plan_create", "fwt_plan_create_split", "fwt_plan_create_tuned",
                 "fwt_execute", "fwt_execute_pass", "fwt_execute_pass_timed",
                 "fwt_execute_check", "fwt_plan_num_passes", "fwt_plan_pass_bits",
                 "fwt_plan_pass_config", "fwt_plan_call_pass_config", "fwt_plan_destroy",
                 "fwt_last_hip_error", "fwt_ablation_workspace", "fwt_ablation_execute",
                 "fwt_ablation_execute_static", "fwt_stream_copy"):
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def _strerror(status):
    return load_library().fwt_strerror(status).decode()


def _int_array(vals):
    if vals is None:
        return None
    return (ctypes.c_int * len(vals))(*[int(v) for v in vals])


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Plan:
    """A plan for 2^n-amplitude vectors of dtype "f32" or "f64".

    ``split`` (bit counts, lowest index bits first) forces a Kronecker
    split; ``eb``/``gbits``/``phases``/``pipe``/``wave`` (one entry per
    pass, -1 = default) force the register-round width, column-group count,
    exchange phases, pipelined kernel and wave-tile kernel of each pass
    (tuning; see fwt_pass_tuning).
    """

    def __init__(self, n, dtype="f32", path=PATH_AUTO, split=None, eb=None, gbits=None,
                 phases=None, pipe=None, wave=None):
        lib = load_library()
        if dtype not in _DTYPES:
            raise ValueError("dtype must be 'f32' or 'f64'")
        self.n, self.dtype = int(n), dtype
        h = ctypes.c_void_p()
        knobs = {"eb": eb, "gbits": gbits, "phases": phases, "pipe": pipe, "wave": wave}
        tuned = any(v is not None for v in knobs.values())
        if split is None and not tuned:
            st = lib.fwt_plan_create(ctypes.byref(h), self.n, _DTYPES[dtype], int(path))
        elif not tuned:
            st = lib.fwt_plan_create_split(ctypes.byref(h), self.n, _DTYPES[dtype],
                                           len(split), _int_array(split))
        else:
            if split is None:
                raise ValueError("tuning needs an explicit split")
            tun = (PassTuning * len(split))()
            for i in range(len(split)):
                for name, vals in knobs.items():
                    setattr(tun[i], name, -1 if vals is None else int(vals[i]))
            st = lib.fwt_plan_create_tuned(ctypes.byref(h), self.n, _DTYPES[dtype],
                                           len(split), _int_array(split), tun)
        if st != FWT_OK:
            raise FwtError(st, "fwt_plan_create(n=%d, %s)" % (self.n, dtype))
        self._h = h

    @property
    def handle(self):
        return self._h

    @property
    def num_passes(self):
        out = ctypes.c_int()
        st = load_library().fwt_plan_num_passes(self._h, ctypes.byref(out))
        if st != FWT_OK:
            raise FwtError(st, "fwt_plan_num_passes")
        return out.value

    @property
    def pass_bits(self):
        out, lib, bits = ctypes.c_int(), load_library(), []
        for i in range(self.num_passes):
            st = lib.fwt_plan_pass_bits(self._h, i, ctypes.byref(out))
            if st != FWT_OK:
                raise FwtError(st, "fwt_plan_pass_bits")
            bits.append(out.value)
        return bits

    def pass_config(self, i, batch=None, with_im=True):
        """Tiling of pass i as a dict (fwt_plan_pass_config); with `batch`,
        the tiling a call on that many vectors launches
        (fwt_plan_call_pass_config)."""
        out = (ctypes.c_int * 12)()
        if batch is None:
            st = load_library().fwt_plan_pass_config(self._h, int(i), out)
        else:
            st = load_library().fwt_plan_call_pass_config(self._h, int(i), int(batch),
                                                           1 if with_im else 0, out)
        if st != FWT_OK:
            raise FwtError(st, "fwt_plan_pass_config")
        keys = ("lo", "bits", "kind", "kr", "eb", "gbits", "phase_bits", "block", "lds",
                "tpw_bits", "pipe", "wave")
        d = dict(zip(keys, list(out)))
        d["kind"] = ("row", "column", "pair", "mfma")[d["kind"]]
        return d

    def kernel_name(self, i, batch=None, with_im=True):
        """Demangled name of pass i's kernel as profilers print it (for a
        call on `batch` vectors when given)."""
        c = self.pass_config(i, batch, with_im)
        if c["kind"] == "pair":
            return "pair_f32_kernel"
        t = "float" if self.dtype == "f32" else "double"
        if c["kind"] == "mfma":
            return "mfma_row_kernel<%s, %d>" % (t, c["bits"])
        if c["wave"] == 2:
            w = c["kr"] - (6 - c["gbits"]) - c["eb"]
            return "lx_kernel<%s, %d, %d, %d, %d, %d, %s>" % (
                t, c["kr"], c["eb"], w, c["phase_bits"], c["gbits"],
                "true" if c["kind"] == "row" else "false")
        if c["wave"]:
            return "wave_kernel<%s, %d, %d, %d, %s>" % (
                t, c["kr"], c["eb"], c["gbits"], "true" if c["kind"] == "row" else "false")
        return "%s<%s, %d, %d, %d, %d, %s>" % (
            "tile_kernel_pipe" if c["pipe"] else "tile_kernel",
            t, c["kr"], c["eb"], c["gbits"], c["phase_bits"],
            "true" if c["kind"] == "row" else "false")

    def _check_tensors(self, re, im):
        """Validate torch tensors for this plan; returns the batch size."""
        return _check_state(re, im, self.n, self.dtype)

    def execute(self, re, im=None, normalize=True, stream=None):
        """Transform torch device tensors re (and im) in place.

        Both must be contiguous, of the plan's dtype, on the current device,
        with numel a multiple of 2^n.  Runs asynchronously on ``stream``
        (default: torch's current stream).
        """
        batch = self._check_tensors(re, im)
        st = load_library().fwt_execute(self._h, batch, self.n, ctypes.c_void_p(re.data_ptr()),
                                        ctypes.c_void_p(im.data_ptr() if im is not None else None),
                                        1 if normalize else 0, _stream_handle(stream))
        if st != FWT_OK:
            raise FwtError(st, "fwt_execute")
        return re, im

    def workspace_size(self, batch, with_im=True):
        """Bytes of workspace execute_ws needs for `batch` vectors: 0 when
        the call runs fwt_execute's passes (see fwt_workspace_size)."""
        out = ctypes.c_size_t()
        st = load_library().fwt_workspace_size(self._h, int(batch), 1 if with_im else 0,
                                                ctypes.byref(out))
        if st != FWT_OK:
            raise FwtError(st, "fwt_workspace_size")
        return out.value

    def execute_ws(self, re, im=None, normalize=True, workspace=None, stream=None):
        """fwt_execute_ws on torch tensors: the one-pass kernel on a device
        workspace (a uint8 tensor of workspace_size bytes) where it applies,
        otherwise fwt_execute."""
        batch = self._check_tensors(re, im)
        wp, wb = _workspace_args(workspace)
        st = load_library().fwt_execute_ws(
            self._h, batch, self.n, ctypes.c_void_p(re.data_ptr()),
            ctypes.c_void_p(im.data_ptr() if im is not None else None), 1 if normalize else 0,
            wp, wb, _stream_handle(stream))
        if st != FWT_OK:
            raise FwtError(st, "fwt_execute_ws")
        return re, im

    def execute_ws_timed(self, re, im, workspace, start, stop, normalize=True, stream=None):
        """execute_ws with torch events recorded by the transform kernel's
        dispatch (see fwt_execute_ws_timed)."""
        import torch
        batch = self._check_tensors(re, im)
        s = torch.cuda.current_stream() if stream is None else stream
        for ev in (start, stop):
            if not ev.cuda_event:
                ev.record(s)
        wp, wb = _workspace_args(workspace)
        st = load_library().fwt_execute_ws_timed(
            self._h, batch, self.n, ctypes.c_void_p(re.data_ptr()),
            ctypes.c_void_p(im.data_ptr() if im is not None else None), 1 if normalize else 0,
            wp, wb, ctypes.c_void_p(s.cuda_stream), ctypes.c_void_p(start.cuda_event),
            ctypes.c_void_p(stop.cuda_event))
        if st != FWT_OK:
            raise FwtError(st, "fwt_execute_ws_timed")

    def bind_ws(self, re, im=None, normalize=True, workspace=None, stream=None):
        """bind() for execute_ws: a zero-argument callable with the
        arguments marshalled once; it keeps the plan, the tensors and the
        workspace alive."""
        batch = self._check_tensors(re, im)
        lib = load_library()
        rp = ctypes.c_void_p(re.data_ptr())
        ip = ctypes.c_void_p(im.data_ptr() if im is not None else None)
        st = lib.fwt_execute_check(self._h, batch, self.n, rp, ip)
        if st != FWT_OK:
            raise FwtError(st, "fwt_execute_check")
        wp, wb = _workspace_args(workspace)
        fn = lib.fwt_execute_ws
        args = (self._h, batch, self.n, rp, ip, 1 if normalize else 0, wp, wb,
                _stream_handle(stream))

        def call():
            st = fn(*args)
            if st != FWT_OK:
                raise FwtError(st, "fwt_execute_ws")
        call.plan = self
        call.tensors = (re, im, workspace)
        return call

    def chunk_vectors(self, batch, with_im=True):
        """Vectors per chunk fwt_execute uses for `batch` vectors (0 = none)."""
        out = ctypes.c_int64()
        st = load_library().fwt_plan_chunk_vectors(self._h, int(batch), 1 if with_im else 0,
                                                   ctypes.byref(out))
        if st != FWT_OK:
            raise FwtError(st, "fwt_plan_chunk_vectors")
        return out.value

    def call_schedule(self, batch, with_im=True):
        """(chunked passes, log2 elements per block, blocks per chunk) of a
        call on `batch` vectors (see fwt_plan_call_schedule)."""
        cp, bb, bl = ctypes.c_int(), ctypes.c_int(), ctypes.c_int64()
        st = load_library().fwt_plan_call_schedule(self._h, int(batch), 1 if with_im else 0,
                                                   ctypes.byref(cp), ctypes.byref(bb),
                                                   ctypes.byref(bl))
        if st != FWT_OK:
            raise FwtError(st, "fwt_plan_call_schedule")
        return cp.value, bb.value, bl.value

    def bind(self, re, im=None, normalize=True, stream=None):
        """A zero-argument callable that enqueues fwt_execute on these
        tensors with the arguments marshalled once (for tight loops).
        Binding validates the arguments (fwt_execute_check) but runs
        nothing; the callable keeps the plan and the bound tensors alive,
        so their memory cannot be handed to another tensor while the
        callable exists."""
        batch = self._check_tensors(re, im)
        lib = load_library()
        rp = ctypes.c_void_p(re.data_ptr())
        ip = ctypes.c_void_p(im.data_ptr() if im is not None else None)
        st = lib.fwt_execute_check(self._h, batch, self.n, rp, ip)
        if st != FWT_OK:
            raise FwtError(st, "fwt_execute_check")
        fn = lib.fwt_execute
        args = (self._h, batch, self.n, rp, ip, 1 if normalize else 0, _stream_handle(stream))
        plan = self

        def call():
            st = fn(*args)
            if st != FWT_OK:
                raise FwtError(st, "fwt_execute")
        call.plan = plan
        call.tensors = (re, im)
        return call

    def execute_pass(self, i, re, im=None, normalize=True, stream=None):
        """Enqueue only pass i (see fwt_execute_pass) on torch tensors."""
        batch = self._check_tensors(re, im)
        st = load_library().fwt_execute_pass(
            self._h, int(i), batch, self.n, ctypes.c_void_p(re.data_ptr()),
            ctypes.c_void_p(im.data_ptr() if im is not None else None),
            1 if normalize else 0, _stream_handle(stream))
        if st != FWT_OK:
            raise FwtError(st, "fwt_execute_pass")
        return re, im

    def execute_pass_timed(self, i, re, im, start, stop, normalize=True, stream=None):
        """Enqueue pass i with torch timing events `start`/`stop` recorded
        by the kernel dispatch itself (see fwt_execute_pass_timed)."""
        import torch
        batch = self._check_tensors(re, im)
        s = torch.cuda.current_stream() if stream is None else stream
        for ev in (start, stop):
            if not ev.cuda_event:          # torch creates events lazily
                ev.record(s)
        st = load_library().fwt_execute_pass_timed(
            self._h, int(i), batch, self.n, ctypes.c_void_p(re.data_ptr()),
            ctypes.c_void_p(im.data_ptr() if im is not None else None), 1 if normalize else 0,
            ctypes.c_void_p(s.cuda_stream), ctypes.c_void_p(start.cuda_event),
            ctypes.c_void_p(stop.cuda_event))
        if st != FWT_OK:
            raise FwtError(st, "fwt_execute_pass_timed")

    def execute_raw(self, batch, re_ptr, im_ptr, normalize, stream_ptr=0):
        """Call fwt_execute on raw device addresses; returns the status."""
        return load_library().fwt_execute(self._h, int(batch), self.n, ctypes.c_void_p(re_ptr),
                                          ctypes.c_void_p(im_ptr), int(normalize),
                                          ctypes.c_void_p(stream_ptr))

    def check_raw(self, batch, re_ptr, im_ptr):
        """Call fwt_execute_check on raw addresses; returns the status."""
        return load_library().fwt_execute_check(self._h, int(batch), self.n,
                                                ctypes.c_void_p(re_ptr), ctypes.c_void_p(im_ptr))

    def close(self):
        if getattr(self, "_h", None):
            load_library().fwt_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _workspace_args(workspace):
    """(pointer, bytes) of a workspace tensor, or (NULL, 0) for None."""
    if workspace is None:
        return ctypes.c_void_p(None), 0
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("the workspace must be a contiguous device tensor")
    return (ctypes.c_void_p(workspace.data_ptr()),
            workspace.numel() * workspace.element_size())


def workspace_status(workspace):
    """Error bits the last one-pass call on `workspace` recorded (0: none);
    synchronise the stream that ran it first (see fwt_workspace_status)."""
    out = ctypes.c_int()
    st = load_library().fwt_workspace_status(ctypes.c_void_p(workspace.data_ptr()),
                                             ctypes.byref(out))
    if st != FWT_OK:
        raise FwtError(st, "fwt_workspace_status")
    return out.value


def execute(re, im=None, n=None, normalize=True, stream=None, path=PATH_AUTO):
    """One-shot transform of the last dimension (2^n) of re/im in place."""
    if n is None:
        N = re.shape[-1]
        n = N.bit_length() - 1
        if (1 << n) != N:
            raise ValueError("last dimension %d is not a power of two" % N)
    dtype = {"torch.float32": "f32", "torch.float64": "f64"}.get(str(re.dtype))
    if dtype is None:
        raise ValueError("re must be float32 or float64")
    return Plan(n, dtype, path).execute(re, im, normalize, stream)


ABLATION_STAGEWISE, ABLATION_POPC_GEMM, ABLATION_MFMA, ABLATION_OZAKI = 1, 2, 3, 4
ABLATION_MFMA_TRANSPOSE = 5


def ablation_workspace(kind, batch, n, dtype="f32", with_im=True):
    """Workspace bytes an ablation needs (see fwt_ablation_workspace)."""
    out = ctypes.c_size_t()
    st = load_library().fwt_ablation_workspace(int(kind), int(batch), int(n), _DTYPES[dtype],
                                               1 if with_im else 0, ctypes.byref(out))
    if st != FWT_OK:
        raise FwtError(st, "fwt_ablation_workspace")
    return out.value


def _check_state(re, im, n, dtype):
    """Validate planar state tensors (dtype "f32"/"f64", vectors of 2^n
    elements); returns the batch size.  Raises ValueError."""
    import torch
    want = torch.float32 if dtype == "f32" else torch.float64
    N = 1 << n
    if re is None:
        raise ValueError("re is required")
    for name, t in (("re", re), ("im", im)):
        if t is None:
            continue
        if t.dtype != want:
            raise ValueError("%s must be %s" % (name, want))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if t.numel() % N:
            raise ValueError("%s.numel() is not a multiple of 2^%d" % (name, n))
    if im is not None and im.numel() != re.numel():
        raise ValueError("re and im must have the same number of elements")
    for name, t in (("re", re), ("im", im)):
        if t is not None and not t.is_cuda:
            raise ValueError("%s must be a device tensor" % name)
    return re.numel() // N


def ablation_execute(kind, re, im=None, n=None, normalize=True, workspace=None, stream=None):
    """Run one of the pages' designs (fwt_ablation_execute) on torch tensors
    in place; `workspace` is a device tensor of at least ablation_workspace
    bytes when the kind needs one."""
    if n is None:
        n = re.shape[-1].bit_length() - 1
    dtype = {"torch.float32": "f32", "torch.float64": "f64"}.get(str(re.dtype))
    if dtype is None:
        raise ValueError("re must be float32 or float64")
    batch = _check_state(re, im, n, dtype)
    if workspace is not None and not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().fwt_ablation_execute(
        int(kind), batch, int(n), _DTYPES[dtype], ctypes.c_void_p(re.data_ptr()),
        ctypes.c_void_p(im.data_ptr() if im is not None else None), 1 if normalize else 0,
        ctypes.c_void_p(ws_ptr), ws_bytes, _stream_handle(stream))
    if st != FWT_OK:
        raise FwtError(st, "fwt_ablation_execute")
    return re, im


def ablation_execute_static(kind, re, im=None, n=None, normalize=True, stream=None):
    """fwt_ablation_execute_static on torch tensors in place: the ablation
    with its workspace in the library's static scratch array (no device
    allocation; raises FwtError with FWT_ESCRATCH when the call needs more
    than STATIC_SCRATCH_BYTES)."""
    if n is None:
        n = re.shape[-1].bit_length() - 1
    dtype = {"torch.float32": "f32", "torch.float64": "f64"}.get(str(re.dtype))
    if dtype is None:
        raise ValueError("re must be float32 or float64")
    batch = _check_state(re, im, n, dtype)
    st = load_library().fwt_ablation_execute_static(
        int(kind), batch, int(n), _DTYPES[dtype], ctypes.c_void_p(re.data_ptr()),
        ctypes.c_void_p(im.data_ptr() if im is not None else None), 1 if normalize else 0,
        _stream_handle(stream))
    if st != FWT_OK:
        raise FwtError(st, "fwt_ablation_execute_static")
    return re, im


def stream_copy(dst, src, stream=None):
    """Copy src to dst (device tensors of equal byte size) with the
    library's streaming copy kernel (measurement aid)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("size mismatch")
    st = load_library().fwt_stream_copy(ctypes.c_void_p(dst.data_ptr()),
                                        ctypes.c_void_p(src.data_ptr()), nbytes,
                                        _stream_handle(stream))
    if st != FWT_OK:
        raise FwtError(st, "fwt_stream_copy")
    return dst
