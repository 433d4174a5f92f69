"""ctypes binding of the CPU comparison GEMV (``cpu/cpu_fused.c``): a
multi-threaded, vectorised host implementation whose epilogue is applied to
each accumulator tile ("ggml-cpu: fuse element-wise epilogues (ADD, MUL,
SILU) into ggml_compute_forward_mul_mat", What).  The benchmark times it
beside the GPU as a CPU baseline; the HIP binding never calls it."""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcpu_fused.so")
FORMATS = {"f32": 0, "f16": 1, "bf16": 2, "q8b32": 3, "q4b32": 4}
ACTS = {"none": 0, "sigmoid": 1, "silu": 2, "silu_mul": 3, "mul": 4, "add": 5}

_LIB = None
_fp = ctypes.POINTER(ctypes.c_float)


def available() -> bool:
    """The library is built for AVX2 + FMA + F16C hosts."""
    flags = open("/proc/cpuinfo").read() if os.path.exists("/proc/cpuinfo") else ""
    return os.path.exists(LIB_PATH) and all(f in flags for f in (" avx2", " fma", " f16c"))


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built (python -m decode_gemv_elementwise_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        lib.cpu_fused_gemv.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, _fp,
                                       ctypes.c_int, _fp, _fp, _fp, ctypes.c_int, ctypes.c_int, _fp]
        lib.cpu_fused_gemv.restype = ctypes.c_int
        lib.cpu_vexp_nonpos.argtypes = [ctypes.c_int64, _fp, _fp]
        lib.cpu_vexp_nonpos.restype = None
        _LIB = lib
    return _LIB


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32).reshape(-1)


def _p(a):
    return None if a is None else a.ctypes.data_as(_fp)


def gemv(fmt, N, K, w, x, act, m=None, r=None, out=None, threads=None, fused=True, acc=None):
    """dst = epilogue(W x) on the host; returns dst (float32 [N]).  out may be
    m or r itself (in place).  Unfused (fused=False), the product is written
    to a separate buffer first (acc, or a fresh one) and the epilogue pass
    reads it, as a GEMV followed by its own element-wise op would."""
    w = np.ascontiguousarray(w).view(np.uint8).reshape(-1)
    x, m, r = _f32(x), _f32(m), _f32(r)
    dst = np.empty(N, np.float32) if out is None else out
    threads = threads or len(os.sched_getaffinity(0))
    if not fused and act != "none" and acc is None:
        acc = np.empty(N, np.float32)
    rc = _lib().cpu_fused_gemv(FORMATS[fmt], N, K, w.ctypes.data, _p(x), ACTS[act], _p(m), _p(r), _p(dst),
                               threads, 1 if fused else 0, _p(acc))
    if rc != 0:
        raise ValueError(f"cpu_fused_gemv rejected {fmt} {N}x{K} act={act}")
    return dst


def vexp_nonpos(x):
    x = _f32(x)
    assert x.size % 8 == 0
    y = np.empty_like(x)
    _lib().cpu_vexp_nonpos(x.size, _p(x), _p(y))
    return y
