"""CPU oracle for the fused decode GEMV -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its
binding) never imports, loads or calls it, and it shares no code with them.

The arithmetic lives in ``gemv_oracle.c`` (plain C, double precision): decode
every weight exactly, accumulate the dot product of each row in double with
the column index ascending, then apply the epilogue as a separate pass.  This
module only marshals numpy arrays into that library, plus the error metric in
``compare.py``.  Formats and epilogues are named by strings here and numbered
by the C file itself.

Sources: "feat(cuda): fuse activations and residual add into mmv f/q
epilogues" (Summary; What changed) for the product and its tails;
"ggml-cpu: fuse element-wise epilogues (ADD, MUL, SILU) into
ggml_compute_forward_mul_mat" (What; Correctness) for the multiply tail and
for the rule that the fused result equals the separate element-wise pass;
"vulkan: fuse the sign multiply into the Hadamard FWHT" (Overview) for the
signed block Hadamard transform that may precede the product.
"""
import ctypes
import os

import numpy as np

from . import build as _build

FORMATS = {"f32": 0, "f16": 1, "bf16": 2, "q8b32": 3, "q4b32": 4}
ACTS = {"none": 0, "sigmoid": 1, "silu": 2, "silu_mul": 3, "mul": 4, "add": 5}

_LIB = None

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_double.restype = ctypes.c_double
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_weight_bytes.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64]
        lib.oracle_weight_bytes.restype = ctypes.c_int64
        lib.oracle_decode_row.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_int64, _dp]
        lib.oracle_decode_row.restype = ctypes.c_int
        lib.oracle_gemv_rows.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, _fp,
                                         ctypes.c_int64, ctypes.c_int64, _dp, _dp, _dp]
        lib.oracle_gemv_rows.restype = ctypes.c_int
        lib.oracle_sigmoid.argtypes = [ctypes.c_double]
        lib.oracle_sigmoid.restype = ctypes.c_double
        lib.oracle_silu.argtypes = [ctypes.c_double]
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_epilogue.argtypes = [ctypes.c_int, ctypes.c_int64, _dp, _fp, _fp, _dp]
        lib.oracle_epilogue.restype = ctypes.c_int
        lib.oracle_glu_epilogue.argtypes = [ctypes.c_int, ctypes.c_int64, _dp, _dp, _dp]
        lib.oracle_glu_epilogue.restype = ctypes.c_int
        lib.oracle_fwht_signed.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _fp, _fp, _dp, _dp]
        lib.oracle_fwht_signed.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _ptr(a, typ):
    return a.ctypes.data_as(typ)


def f16_to_double(bits: int) -> float:
    return _lib().oracle_f16_to_double(int(bits))


def bf16_to_double(bits: int) -> float:
    return _lib().oracle_bf16_to_double(int(bits))


def sigmoid(a: float) -> float:
    return _lib().oracle_sigmoid(float(a))


def silu(a: float) -> float:
    return _lib().oracle_silu(float(a))


def weight_bytes(fmt: str, N: int, K: int) -> int:
    return int(_lib().oracle_weight_bytes(FORMATS[fmt], N, K))


def _check_w(fmt, N, K, w):
    nb = weight_bytes(fmt, N, K)
    if nb < 0:
        raise ValueError(f"invalid matrix {fmt} {N}x{K}")
    w = np.ascontiguousarray(w).view(np.uint8).reshape(-1)
    if w.size < nb:
        raise ValueError(f"weight buffer holds {w.size} bytes, {fmt} {N}x{K} needs {nb}")
    return w


def decode(fmt: str, N: int, K: int, w: np.ndarray, rows=None) -> np.ndarray:
    """Exact values of rows [begin, end) of W as float64 [rows, K]."""
    w = _check_w(fmt, N, K, w)
    b, e = (0, N) if rows is None else rows
    out = np.empty((e - b, K), dtype=np.float64)
    for i in range(b, e):
        rc = _lib().oracle_decode_row(FORMATS[fmt], N, K, w.ctypes.data, i, _ptr(out[i - b], _dp))
        if rc != 0:
            raise ValueError("oracle_decode_row failed")
    return out


def gemv(fmt: str, N: int, K: int, w: np.ndarray, x: np.ndarray, rows=None):
    """(acc, absacc) for rows [begin, end): acc_i = sum_j w_ij x_j, absacc_i =
    sum_j |w_ij x_j|, both float64, accumulated in double with j ascending."""
    w = _check_w(fmt, N, K, w)
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.shape != (K,):
        raise ValueError("x must hold K float32 values")
    b, e = (0, N) if rows is None else rows
    acc = np.empty(e - b, dtype=np.float64)
    absacc = np.empty(e - b, dtype=np.float64)
    rowbuf = np.empty(K, dtype=np.float64)
    rc = _lib().oracle_gemv_rows(FORMATS[fmt], N, K, w.ctypes.data, _ptr(x, _fp), b, e,
                                 _ptr(acc, _dp), _ptr(absacc, _dp), _ptr(rowbuf, _dp))
    if rc != 0:
        raise ValueError("oracle_gemv_rows failed")
    return acc, absacc


def epilogue(act: str, acc: np.ndarray, m=None, r=None) -> np.ndarray:
    """y = act(acc) as its own pass; m and r are the float32 operands."""
    acc = np.ascontiguousarray(acc, dtype=np.float64).reshape(-1)
    n = acc.size
    mp = rp = None
    if m is not None:
        m = np.ascontiguousarray(m, dtype=np.float32).reshape(-1)
        assert m.size == n
        mp = _ptr(m, _fp)
    if r is not None:
        r = np.ascontiguousarray(r, dtype=np.float32).reshape(-1)
        assert r.size == n
        rp = _ptr(r, _fp)
    y = np.empty(n, dtype=np.float64)
    rc = _lib().oracle_epilogue(ACTS[act], n, _ptr(acc, _dp), mp, rp, _ptr(y, _dp))
    if rc != 0:
        raise ValueError(f"oracle_epilogue failed for act={act}")
    return y


def reference(fmt, N, K, w, x, act, m=None, r=None, rows=None):
    """Full oracle for one call: (y, acc, absacc) over rows [begin, end);
    m and r are given for all N rows and sliced here."""
    b, e = (0, N) if rows is None else rows
    acc, absacc = gemv(fmt, N, K, w, x, rows=(b, e))
    ms = None if m is None else np.asarray(m, dtype=np.float32).reshape(-1)[b:e]
    rs = None if r is None else np.asarray(r, dtype=np.float32).reshape(-1)[b:e]
    return epilogue(act, acc, ms, rs), acc, absacc


def glu_epilogue(act: str, g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """y = act(g) * u as its own pass (act: "silu" or "sigmoid"), in double."""
    g = np.ascontiguousarray(g, dtype=np.float64).reshape(-1)
    u = np.ascontiguousarray(u, dtype=np.float64).reshape(-1)
    assert g.size == u.size
    y = np.empty(g.size, dtype=np.float64)
    rc = _lib().oracle_glu_epilogue(ACTS[act], g.size, _ptr(g, _dp), _ptr(u, _dp), _ptr(y, _dp))
    if rc != 0:
        raise ValueError(f"oracle_glu_epilogue failed for act={act}")
    return y


def glu_reference(fmt, N, K, w_gate, w_up, x, act="silu", rows=None):
    """Gated pair: (y, g, absg, u, absu) over rows [begin, end), where g and u
    are the gate and up row sums and y = act(g) * u."""
    g, ag = gemv(fmt, N, K, w_gate, x, rows=rows)
    u, au = gemv(fmt, N, K, w_up, x, rows=rows)
    return glu_epilogue(act, g, u), g, ag, u, au


def ncols_reference(fmt, N, K, w, X, act, M=None, R=None, rows=None):
    """Several destination columns over one W: column b is the one-column
    product of x_b = X[b] followed by the epilogue with the operand rows
    M[b] / R[b].  The matrix-vector fusion of "feat(cuda): fuse activations
    and residual add into mmv f/q epilogues" (Summary) is stated for one
    destination column; this is its plain widening to ncols columns, each
    column computed exactly as a separate one-column call.

    X is float32 [ncols, K]; M and R are float32 [ncols, N] (or None).
    Returns (Y, acc, absacc), each float64 [ncols, rows], row b of each being
    destination column b (the b-major layout dst[b * N + i])."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    if X.ndim != 2 or X.shape[1] != K:
        raise ValueError("X must be float32 [ncols, K]")
    B = X.shape[0]
    b0, e0 = (0, N) if rows is None else rows
    Y = np.empty((B, e0 - b0))
    acc = np.empty((B, e0 - b0))
    absacc = np.empty((B, e0 - b0))
    for b in range(B):
        mb = None if M is None else np.asarray(M, dtype=np.float32).reshape(B, N)[b]
        rb = None if R is None else np.asarray(R, dtype=np.float32).reshape(B, N)[b]
        Y[b], acc[b], absacc[b] = reference(fmt, N, K, w, X[b], act, m=mb, r=rb, rows=(b0, e0))
    return Y, acc, absacc


def glu_ncols_reference(fmt, N, K, w_gate, w_up, X, act="silu", rows=None):
    """The gated pair over several destination columns: column b is the
    one-column gated pair of x_b = X[b], y_b = act(W_gate x_b) * (W_up x_b).
    The gate path of "feat(cuda): fuse activations and residual add into mmv
    f/q epilogues" (Summary) is stated for one destination column; this is
    its plain widening to ncols columns, each column computed exactly as a
    separate one-column call.

    X is float32 [ncols, K].  Returns (Y, G, absG, U, absU), each float64
    [ncols, rows]; row b of each is destination column b (dst[b * N + i])."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    if X.ndim != 2 or X.shape[1] != K:
        raise ValueError("X must be float32 [ncols, K]")
    B = X.shape[0]
    b0, e0 = (0, N) if rows is None else rows
    out = [np.empty((B, e0 - b0)) for _ in range(5)]
    for b in range(B):
        res = glu_reference(fmt, N, K, w_gate, w_up, X[b], act, rows=(b0, e0))
        for o, v in zip(out, res):
            o[b] = v
    return tuple(out)


def fwht_signed(x, s, n):
    """Signed Hadamard transform of every row of x ([K] or [rows, K] float32):
    y = n^-1/2 H_n (x * s) per block of n, the sign of element k being
    s[k mod len(s)] ("vulkan: fuse the sign multiply into the Hadamard FWHT",
    Overview; Sylvester order and the orthonormal scale are the readings
    stated in gemv_oracle.c).  Returns (y, d) in float64 with x's shape, d
    being n^-1/2 sum |x s| over each output's block."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    s = np.ascontiguousarray(s, dtype=np.float32).reshape(-1)
    rows = x.reshape(-1, x.shape[-1])
    K = rows.shape[1]
    y = np.empty(rows.shape)
    d = np.empty(rows.shape)
    for i in range(rows.shape[0]):
        xi = np.ascontiguousarray(rows[i])
        rc = _lib().oracle_fwht_signed(n, K, s.size, _ptr(xi, _fp), _ptr(s, _fp), _ptr(y[i], _dp), _ptr(d[i], _dp))
        if rc != 0:
            raise ValueError(f"invalid signed FWHT: n={n} K={K} len(s)={s.size}")
    return y.reshape(x.shape), d.reshape(x.shape)


def fwht_gemv_reference(fmt, N, K, w, x, s, n, act, m=None, r=None, rows=None):
    """The product after the signed transform, as the unfused graph computes
    it: x' = fwht_signed(x, s, n) rounded to float32 (the transform's output is
    a float32 tensor), then reference(fmt, N, K, w, x', act, m, r).  Returns
    (y, acc, absacc) where absacc also carries sum_j |w_ij| d_j, the way the
    transform's own rounding reaches row i."""
    xp, d = fwht_signed(x, s, n)
    y, acc, absacc = reference(fmt, N, K, w, xp.astype(np.float32), act, m=m, r=r, rows=rows)
    _, absd = gemv(fmt, N, K, w, d.astype(np.float32), rows=rows)
    return y, acc, absacc + absd
