"""ctypes binding of the C ABI in ``include/gemv_fused.h``.

Argument marshalling only: every step of the computation runs in the HIP
library.  Functions carry the C names.  Tensors are torch tensors (device
memory) or, for the host-only checks, raw integer addresses with explicit
shapes.  There is no fallback: if ``libgemv_fused.so`` is missing, loading
fails with an error that says how to build it.
"""
import ctypes
import functools
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgemv_fused.so")

FORMATS = {"f32": 0, "f16": 1, "bf16": 2, "q8b32": 3, "q4b32": 4}
ACTS = {"none": 0, "sigmoid": 1, "silu": 2, "silu_mul": 3, "mul": 4, "add": 5}
STATUS = {0: "GEMV_OK", -1: "GEMV_E_NULL", -2: "GEMV_E_DIM", -3: "GEMV_E_FMT", -4: "GEMV_E_ACT",
          -5: "GEMV_E_OPERAND", -6: "GEMV_E_LAYOUT", -7: "GEMV_E_ALIAS", -8: "GEMV_E_ALIGN", -9: "GEMV_E_HIP"}
STATUS_CODE = {v: k for k, v in STATUS.items()}
MAX_DIMS = 4


class GemvView(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * MAX_DIMS), ("stride", ctypes.c_int64 * MAX_DIMS)]


class GemvError(RuntimeError):
    def __init__(self, status, message, hip_error=0):
        super().__init__(f"{STATUS.get(status, status)}: {message}"
                         + (f" (hipError {hip_error})" if hip_error else ""))
        self.status = status
        self.hip_error = hip_error


_LIB = None
_VP = ctypes.c_void_p
_I64 = ctypes.c_int64
_VIEWP = ctypes.POINTER(GemvView)


def load(path=None):
    """Load libgemv_fused.so (build it with ``python -m decode_gemv_elementwise_amd.build``).
    ``path`` selects another build of the same library (the first load wins)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m decode_gemv_elementwise_amd.build` "
                          "(or __graft_entry__.build()) first")
    # The library needs libamdhip64.so.7 and binds to whichever copy the
    # process maps first; torch ships its own.  Importing torch first makes
    # the library and torch share torch's HIP runtime (one runtime per
    # process, the configuration every test runs in).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    lib.gemv_fused.argtypes = [_VP, ctypes.c_int, _I64, _I64, _VP, ctypes.c_int, _VIEWP, _VIEWP, _VIEWP, _VP]
    lib.gemv_fused.restype = ctypes.c_int
    lib.gemv_validate.argtypes = [_VP, ctypes.c_int, _I64, _I64, _VP, ctypes.c_int, _VIEWP, _VIEWP, _VIEWP]
    lib.gemv_validate.restype = ctypes.c_int
    lib.gemv_epilogue.argtypes = [ctypes.c_int, _I64, _VP, _VIEWP, _VIEWP, _VIEWP, _VP]
    lib.gemv_epilogue.restype = ctypes.c_int
    lib.gemv_epilogue_validate.argtypes = [ctypes.c_int, _I64, _VP, _VIEWP, _VIEWP, _VIEWP]
    lib.gemv_epilogue_validate.restype = ctypes.c_int
    lib.gemv_glu.argtypes = [_VP, _VP, ctypes.c_int, _I64, _I64, _VP, ctypes.c_int, _VIEWP, _VP]
    lib.gemv_glu.restype = ctypes.c_int
    lib.gemv_glu_validate.argtypes = [_VP, _VP, ctypes.c_int, _I64, _I64, _VP, ctypes.c_int, _VIEWP]
    lib.gemv_glu_validate.restype = ctypes.c_int
    lib.gemv_glu_ncols.argtypes = [_VP, _VP, ctypes.c_int, _I64, _I64, _I64, _VP, ctypes.c_int, _VIEWP, _VP]
    lib.gemv_glu_ncols.restype = ctypes.c_int
    lib.gemv_glu_ncols_validate.argtypes = [_VP, _VP, ctypes.c_int, _I64, _I64, _I64, _VP, ctypes.c_int, _VIEWP]
    lib.gemv_glu_ncols_validate.restype = ctypes.c_int
    lib.gemv_fused_ncols.argtypes = [_VP, ctypes.c_int, _I64, _I64, _I64, _VP, ctypes.c_int, _VIEWP, _VIEWP,
                                     _VIEWP, _VP]
    lib.gemv_fused_ncols.restype = ctypes.c_int
    lib.gemv_fused_ncols_validate.argtypes = [_VP, ctypes.c_int, _I64, _I64, _I64, _VP, ctypes.c_int, _VIEWP,
                                              _VIEWP, _VIEWP]
    lib.gemv_fused_ncols_validate.restype = ctypes.c_int
    lib.gemv_ncols_kernel.argtypes = [ctypes.c_int, _I64, _I64, _I64]
    lib.gemv_ncols_kernel.restype = ctypes.c_int
    lib.gemv_fwht_signed.argtypes = [_VP, _VP, _I64, _I64, _I64, _I64, _VP, _VP]
    lib.gemv_fwht_signed.restype = ctypes.c_int
    lib.gemv_fwht_signed_validate.argtypes = [_VP, _VP, _I64, _I64, _I64, _I64, _VP]
    lib.gemv_fwht_signed_validate.restype = ctypes.c_int
    lib.gemv_fused_fwht.argtypes = [_VP, ctypes.c_int, _I64, _I64, _VP, _VP, _I64, _I64, ctypes.c_int, _VIEWP,
                                    _VIEWP, _VIEWP, _VP]
    lib.gemv_fused_fwht.restype = ctypes.c_int
    lib.gemv_fused_fwht_validate.argtypes = [_VP, ctypes.c_int, _I64, _I64, _VP, _VP, _I64, _I64, ctypes.c_int,
                                             _VIEWP, _VIEWP, _VIEWP]
    lib.gemv_fused_fwht_validate.restype = ctypes.c_int
    lib.gemv_weight_bytes.argtypes = [ctypes.c_int, _I64, _I64]
    lib.gemv_weight_bytes.restype = _I64
    lib.gemv_strerror.argtypes = [ctypes.c_int]
    lib.gemv_strerror.restype = ctypes.c_char_p
    lib.gemv_last_hip_error.argtypes = []
    lib.gemv_last_hip_error.restype = ctypes.c_int
    _LIB = lib
    return lib


# ------------------------------------------------------------------ marshalling

def _addr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def make_view(data, shape=None, stride=None) -> GemvView:
    """A GemvView from a torch tensor (f32), or from an address plus shape and
    strides (in elements; C-contiguous strides by default)."""
    if not isinstance(data, int):
        import torch
        if data.dtype != torch.float32:
            raise TypeError("epilogue operands and dst are float32")
        shape = tuple(data.shape) if shape is None else tuple(shape)
        stride = tuple(data.stride()) if stride is None else tuple(stride)
        if len(shape) == 0:
            shape, stride = (1,), (1,)
        data = data.data_ptr()
    shape = tuple(shape)
    if stride is None:
        st, acc = [], 1
        for s in reversed(shape):
            st.append(acc)
            acc *= s
        stride = tuple(reversed(st))
    if not 1 <= len(shape) <= MAX_DIMS or len(stride) != len(shape):
        # pass the rank through unchanged so the library reports the layout error
        v = GemvView()
        v.data = data
        v.ndim = len(shape)
        for i, (s, t) in enumerate(list(zip(shape, stride))[:MAX_DIMS]):
            v.shape[i], v.stride[i] = s, t
        return v
    v = GemvView()
    v.data = data
    v.ndim = len(shape)
    for i, (s, t) in enumerate(zip(shape, stride)):
        v.shape[i] = s
        v.stride[i] = t
    return v


def _as_view(v):
    if v is None:
        return None
    if isinstance(v, GemvView):
        return ctypes.pointer(v)
    return ctypes.pointer(make_view(v))


# ------------------------------------------------------------------ tensor checks of the launching calls
# A launch hands raw addresses to kernels, so a host tensor, a tensor on
# another device, a wrong dtype or a buffer shorter than what the kernel reads
# would become an out-of-bounds or host-address access on the GPU.  Every torch
# tensor given to a launching call is checked here first; raw integer addresses
# are the caller's responsibility.  The library's own checks (shapes, formats,
# overlaps) still follow in C.

def _check_tensor(t, name, dtype=None, min_bytes=None, tensors=None):
    """Address of t after checking its dtype, contiguity and size (None and
    int addresses pass through); t joins `tensors`, whose devices
    _check_devices checks once every argument has passed these checks."""
    import torch
    if t is None or isinstance(t, int):
        return t
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor or an integer address, got {type(t).__name__}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise TypeError(f"{name} must be contiguous")
    nbytes = t.numel() * t.element_size()
    if min_bytes is not None and min_bytes > 0 and nbytes < min_bytes:
        raise ValueError(f"{name} holds {nbytes} bytes, the call reads {min_bytes}")
    if tensors is not None:
        tensors.append((name, t))
    return t.data_ptr()


def _check_view_tensor(v, name, tensors):
    """An operand or dst given as a tensor joins the device check (its shape,
    layout and overlap checks are the library's)."""
    import torch
    if isinstance(v, torch.Tensor):
        if v.dtype != torch.float32:
            raise TypeError(f"{name} must be torch.float32, got {v.dtype}")
        tensors.append((name, v))


def _check_devices(tensors):
    """Every tensor on the GPU, all on the current device."""
    import torch
    devs = set()
    for name, t in tensors:
        if not t.is_cuda:
            raise TypeError(f"{name}: tensor arguments of a launching call must be on the GPU")
        devs.add(t.device.index)
    if not devs:
        return
    if len(devs) > 1:
        raise TypeError(f"tensor arguments are on different GPUs: {sorted(devs)}")
    cur = torch.cuda.current_device()
    if devs != {cur}:
        raise TypeError(f"tensor arguments are on cuda:{devs.pop()}, the current device is cuda:{cur}")


@functools.lru_cache(maxsize=512)
def _weight_bytes_of(code, N, K):
    return int(load().gemv_weight_bytes(code, N, K))


def _weight_bytes_or_none(wfmt, N, K):
    try:
        b = _weight_bytes_of(_fmt(wfmt), N, K)
    except (KeyError, TypeError, ctypes.ArgumentError):
        return None
    return b if b > 0 else None


def _checked_product_args(W, wfmt, N, K, x, x_floats, views, W2=None):
    """Checked addresses of W (and W2) and x for a product over x_floats
    values of x; views are the operand / dst arguments."""
    import torch
    devices = []
    wb = _weight_bytes_or_none(wfmt, N, K)
    w = _check_tensor(W, "W", min_bytes=wb, tensors=devices)
    w2 = _check_tensor(W2, "W_up", min_bytes=wb, tensors=devices)
    xa = _check_tensor(x, "x", dtype=torch.float32,
                       min_bytes=4 * x_floats if isinstance(x_floats, int) and x_floats > 0 else None,
                       tensors=devices)
    for name, v in views.items():
        _check_view_tensor(v, name, devices)
    _check_devices(devices)
    return w, w2, xa


def _fmt(wfmt):
    return FORMATS[wfmt] if isinstance(wfmt, str) else int(wfmt)


def _act(act):
    return ACTS[act] if isinstance(act, str) else int(act)


_CURRENT_STREAM = None  # resolved on first use: () -> handle of the current stream


def _current_stream_handle():
    """The raw handle of the current device's current stream.  torch's
    torch.cuda.current_stream() builds a Stream object per call (about 2.8 us,
    as long as the launch itself); where torch exposes the raw query, that is
    used instead (about 0.2 us) with the same result."""
    global _CURRENT_STREAM
    if _CURRENT_STREAM is None:
        import torch
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        dev = getattr(torch._C, "_cuda_getDevice", None)
        if raw is not None and dev is not None:
            _CURRENT_STREAM = lambda: raw(dev())
        else:
            _CURRENT_STREAM = lambda: torch.cuda.current_stream().cuda_stream
    return _CURRENT_STREAM()


def _stream(stream):
    if stream is None:
        return _current_stream_handle()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _raise(status):
    lib = load()
    raise GemvError(status, lib.gemv_strerror(status).decode(),
                    lib.gemv_last_hip_error() if status == STATUS_CODE["GEMV_E_HIP"] else 0)


def _ncols_floats(ncols, K):
    """x values a several-column call reads, or None where the library itself
    rejects the column count (1..8) or K."""
    if isinstance(ncols, int) and isinstance(K, int) and 1 <= ncols <= 8 and K > 0:
        return ncols * K
    return None


def _int_or_none(v):
    return v if isinstance(v, int) and v > 0 else None


def _checked_fwht_args(x, signs, nrows, K, nsigns, dst):
    import torch
    devices = []
    nx = nrows * K if _int_or_none(nrows) and _int_or_none(K) else None
    xa = _check_tensor(x, "x", dtype=torch.float32, min_bytes=4 * nx if nx else None, tensors=devices)
    sa = _check_tensor(signs, "signs", dtype=torch.float32,
                       min_bytes=4 * nsigns if _int_or_none(nsigns) else None, tensors=devices)
    da = _check_tensor(dst, "dst", dtype=torch.float32, min_bytes=4 * nx if nx else None, tensors=devices)
    _check_devices(devices)
    return xa, sa, da


def _checked_fused_fwht_args(W, wfmt, N, K, x, signs, nsigns, mul_operand, add_operand, dst):
    import torch
    w, _, _ = _checked_product_args(W, wfmt, N, K, x, K, {"mul_operand": mul_operand, "add_operand": add_operand,
                                                          "dst": dst})
    devices = []
    _check_view_tensor(x, "x", devices)
    sa = _check_tensor(signs, "signs", dtype=torch.float32,
                       min_bytes=4 * nsigns if _int_or_none(nsigns) else None, tensors=devices)
    _check_devices(devices)
    return w, sa


# ------------------------------------------------------------------ API (C names)

def gemv_fused(W, wfmt, N, K, x, act, mul_operand=None, add_operand=None, dst=None, stream=None):
    """dst = epilogue(W x) on the GPU (one launch, asynchronous on ``stream``;
    default: torch's current stream).  Raises GemvError on a rejected call."""
    w, _, xa = _checked_product_args(W, wfmt, N, K, x, K, {"mul_operand": mul_operand, "add_operand": add_operand,
                                                            "dst": dst})
    st = load().gemv_fused(w, _fmt(wfmt), N, K, xa, _act(act), _as_view(mul_operand),
                           _as_view(add_operand), _as_view(dst), _stream(stream))
    if st != 0:
        _raise(st)


def gemv_validate(W, wfmt, N, K, x, act, mul_operand=None, add_operand=None, dst=None) -> int:
    """Host-only checks; returns the status code (no HIP call)."""
    return load().gemv_validate(_addr(W), _fmt(wfmt), N, K, _addr(x), _act(act), _as_view(mul_operand),
                                _as_view(add_operand), _as_view(dst))


def gemv_epilogue(act, N, acc, mul_operand=None, add_operand=None, dst=None, stream=None):
    """dst = epilogue(acc) as a separate pass (the unfused path)."""
    import torch
    devices = []
    a = _check_tensor(acc, "acc", dtype=torch.float32,
                      min_bytes=4 * N if isinstance(N, int) and N > 0 else None, tensors=devices)
    for name, v in (("mul_operand", mul_operand), ("add_operand", add_operand), ("dst", dst)):
        _check_view_tensor(v, name, devices)
    _check_devices(devices)
    st = load().gemv_epilogue(_act(act), N, a, _as_view(mul_operand), _as_view(add_operand),
                              _as_view(dst), _stream(stream))
    if st != 0:
        _raise(st)


def gemv_epilogue_validate(act, N, acc, mul_operand=None, add_operand=None, dst=None) -> int:
    return load().gemv_epilogue_validate(_act(act), N, _addr(acc), _as_view(mul_operand),
                                         _as_view(add_operand), _as_view(dst))


def gemv_glu(W_gate, W_up, wfmt, N, K, x, act="silu", dst=None, stream=None):
    """dst = act(W_gate x) * (W_up x) in one launch (act: "silu" or "sigmoid")."""
    wg, wu, xa = _checked_product_args(W_gate, wfmt, N, K, x, K, {"dst": dst}, W2=W_up)
    st = load().gemv_glu(wg, wu, _fmt(wfmt), N, K, xa, _act(act), _as_view(dst), _stream(stream))
    if st != 0:
        _raise(st)


def gemv_glu_validate(W_gate, W_up, wfmt, N, K, x, act="silu", dst=None) -> int:
    return load().gemv_glu_validate(_addr(W_gate), _addr(W_up), _fmt(wfmt), N, K, _addr(x), _act(act),
                                    _as_view(dst))


def gemv_glu_ncols(W_gate, W_up, wfmt, N, K, ncols, x, act="silu", dst=None, stream=None):
    """dst[b, i] = act((W_gate x_b)_i) * (W_up x_b)_i for ncols columns x_b =
    x[b] (x: [ncols, K] f32; dst: ncols * N f32 in [ncols][N] order), one launch."""
    wg, wu, xa = _checked_product_args(W_gate, wfmt, N, K, x, _ncols_floats(ncols, K), {"dst": dst}, W2=W_up)
    st = load().gemv_glu_ncols(wg, wu, _fmt(wfmt), N, K, ncols, xa, _act(act), _as_view(dst), _stream(stream))
    if st != 0:
        _raise(st)


def gemv_glu_ncols_validate(W_gate, W_up, wfmt, N, K, ncols, x, act="silu", dst=None) -> int:
    return load().gemv_glu_ncols_validate(_addr(W_gate), _addr(W_up), _fmt(wfmt), N, K, ncols, _addr(x), _act(act),
                                          _as_view(dst))


def gemv_fused_ncols(W, wfmt, N, K, ncols, x, act, mul_operand=None, add_operand=None, dst=None, stream=None):
    """dst[b, i] = epilogue((W x_b)_i) for ncols columns x_b = x[b] (x: [ncols, K]
    f32; dst and operands: ncols * N f32 in [ncols][N] order), one launch."""
    w, _, xa = _checked_product_args(W, wfmt, N, K, x, _ncols_floats(ncols, K), {"mul_operand": mul_operand,
                                                            "add_operand": add_operand, "dst": dst})
    st = load().gemv_fused_ncols(w, _fmt(wfmt), N, K, ncols, xa, _act(act), _as_view(mul_operand),
                                 _as_view(add_operand), _as_view(dst), _stream(stream))
    if st != 0:
        _raise(st)


def gemv_fused_ncols_validate(W, wfmt, N, K, ncols, x, act, mul_operand=None, add_operand=None, dst=None) -> int:
    return load().gemv_fused_ncols_validate(_addr(W), _fmt(wfmt), N, K, ncols, _addr(x), _act(act),
                                            _as_view(mul_operand), _as_view(add_operand), _as_view(dst))


NCOLS_KERNELS = {1: "one_column", 2: "columns", 3: "columns_generic", 4: "columns_matrix"}


def gemv_ncols_kernel(wfmt, N, K, ncols) -> str:
    """Name of the kernel gemv_fused_ncols takes for this format and shape on
    the current device ('one_column', 'columns', 'columns_generic',
    'columns_matrix'); GemvError for arguments it would reject."""
    st = load().gemv_ncols_kernel(_fmt(wfmt), N, K, ncols)
    if st < 0:
        _raise(st)
    return NCOLS_KERNELS[st]


def gemv_fwht_signed(x, signs, nrows, K, n, nsigns, dst, stream=None):
    """dst = n^-1/2 H_n (x * s) per block of n, for nrows rows of K f32 values."""
    xa, sa, da = _checked_fwht_args(x, signs, nrows, K, nsigns, dst)
    st = load().gemv_fwht_signed(xa, sa, nrows, K, n, nsigns, da, _stream(stream))
    if st != 0:
        _raise(st)


def gemv_fwht_signed_validate(x, signs, nrows, K, n, nsigns, dst) -> int:
    return load().gemv_fwht_signed_validate(_addr(x), _addr(signs), nrows, K, n, nsigns, _addr(dst))


def gemv_fused_fwht(W, wfmt, N, K, x, signs, n, nsigns, act, mul_operand=None, add_operand=None, dst=None,
                    stream=None):
    """dst = epilogue(W . FWHT_n(x * s)) in one launch."""
    w, sa = _checked_fused_fwht_args(W, wfmt, N, K, x, signs, nsigns, mul_operand, add_operand, dst)
    st = load().gemv_fused_fwht(w, _fmt(wfmt), N, K, _addr(x), sa, n, nsigns, _act(act),
                                _as_view(mul_operand), _as_view(add_operand), _as_view(dst), _stream(stream))
    if st != 0:
        _raise(st)


def gemv_fused_fwht_validate(W, wfmt, N, K, x, signs, n, nsigns, act, mul_operand=None, add_operand=None,
                             dst=None) -> int:
    return load().gemv_fused_fwht_validate(_addr(W), _fmt(wfmt), N, K, _addr(x), _addr(signs), n, nsigns,
                                           _act(act), _as_view(mul_operand), _as_view(add_operand), _as_view(dst))


def gemv_weight_bytes(wfmt, N, K) -> int:
    return int(load().gemv_weight_bytes(_fmt(wfmt), N, K))


def gemv_strerror(status: int) -> str:
    return load().gemv_strerror(status).decode()


def gemv_last_hip_error() -> int:
    return int(load().gemv_last_hip_error())


class PreparedGlu:
    """A gemv_glu call with its dst view marshalled once."""

    def __init__(self, W_gate, W_up, wfmt, N, K, x, act="silu", dst=None):
        self._lib = load()
        wg, wu, xa = _checked_product_args(W_gate, wfmt, N, K, x, K, {"dst": dst}, W2=W_up)
        self._view = dst if isinstance(dst, GemvView) else make_view(dst)
        self._ptr = ctypes.pointer(self._view)
        self._args = (wg, wu, _fmt(wfmt), N, K, xa, _act(act))

    def __call__(self, stream=None):
        st = self._lib.gemv_glu(*self._args, self._ptr, _stream(stream))
        if st != 0:
            _raise(st)


class PreparedGluNcols:
    """A gemv_glu_ncols call with its dst view marshalled once."""

    def __init__(self, W_gate, W_up, wfmt, N, K, ncols, x, act="silu", dst=None):
        self._lib = load()
        wg, wu, xa = _checked_product_args(W_gate, wfmt, N, K, x, _ncols_floats(ncols, K), {"dst": dst}, W2=W_up)
        self._view = make_view(dst)
        self._ptr = ctypes.pointer(self._view)
        self._args = (wg, wu, _fmt(wfmt), N, K, ncols, xa, _act(act))

    def __call__(self, stream=None):
        st = self._lib.gemv_glu_ncols(*self._args, self._ptr, _stream(stream))
        if st != 0:
            _raise(st)


class PreparedCall:
    """A gemv_fused call with its views marshalled once, for tight loops and
    graph capture (the tensors must stay alive and in place)."""

    def __init__(self, W, wfmt, N, K, x, act, mul_operand=None, add_operand=None, dst=None, _x_floats=None):
        self._lib = load()
        _checked_product_args(W, wfmt, N, K, x, K if _x_floats is None else (_x_floats or None),
                              {"mul_operand": mul_operand, "add_operand": add_operand, "dst": dst})
        self._views = [None if v is None else (v if isinstance(v, GemvView) else make_view(v))
                       for v in (mul_operand, add_operand, dst)]
        self._ptrs = [None if v is None else ctypes.pointer(v) for v in self._views]
        self._args = (_addr(W), _fmt(wfmt), N, K, _addr(x), _act(act))

    def __call__(self, stream=None):
        st = self._lib.gemv_fused(*self._args, *self._ptrs, _stream(stream))
        if st != 0:
            _raise(st)


class PreparedNcols(PreparedCall):
    """A gemv_fused_ncols call with its views marshalled once."""

    def __init__(self, W, wfmt, N, K, ncols, x, act, mul_operand=None, add_operand=None, dst=None):
        super().__init__(W, wfmt, N, K, x, act, mul_operand, add_operand, dst, _x_floats=_ncols_floats(ncols, K))
        self._args = (_addr(W), _fmt(wfmt), N, K, ncols, _addr(x), _act(act))

    def __call__(self, stream=None):
        st = self._lib.gemv_fused_ncols(*self._args, *self._ptrs, _stream(stream))
        if st != 0:
            _raise(st)


class PreparedFusedFwht(PreparedCall):
    """A gemv_fused_fwht call with its views marshalled once."""

    def __init__(self, W, wfmt, N, K, x, signs, n, nsigns, act, mul_operand=None, add_operand=None, dst=None):
        super().__init__(W, wfmt, N, K, x, act, mul_operand, add_operand, dst)
        _checked_fused_fwht_args(W, wfmt, N, K, x, signs, nsigns, mul_operand, add_operand, dst)
        self._args = (_addr(W), _fmt(wfmt), N, K, _addr(x), _addr(signs), n, nsigns, _act(act))

    def __call__(self, stream=None):
        st = self._lib.gemv_fused_fwht(*self._args, *self._ptrs, _stream(stream))
        if st != 0:
            _raise(st)


class PreparedFwht:
    """A gemv_fwht_signed call with its arguments marshalled once."""

    def __init__(self, x, signs, nrows, K, n, nsigns, dst):
        self._lib = load()
        xa, sa, da = _checked_fwht_args(x, signs, nrows, K, nsigns, dst)
        self._args = (xa, sa, nrows, K, n, nsigns, da)

    def __call__(self, stream=None):
        st = self._lib.gemv_fwht_signed(*self._args, _stream(stream))
        if st != 0:
            _raise(st)
