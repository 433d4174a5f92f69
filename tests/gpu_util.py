"""Helpers for the GPU tests: device copies, one fused call, the oracle beside it."""
import numpy as np
import torch

import oracle
from oracle.compare import TOLERANCE, compare, health_bound
from decode_gemv_elementwise_amd import binding

# Values per 16-byte chunk of W, per format.
CHUNK_VALUES = {"f32": 4, "f16": 8, "bf16": 8, "q8b32": 16, "q4b32": 32}


def lane_depth(fmt, K):
    """Chained float32 roundings between the products and one output on the
    vector-ALU kernels: a lane sums its ceil(K / (64 E)) chunks in order, each
    chunk a chain of E products plus the fold and the scale (2 more), and the
    64 lane sums meet in a 6-level tree."""
    E = CHUNK_VALUES[fmt]
    return -(-K // (64 * E)) * (E + 2) + 6


def assert_healthy(res, fmt, K, tag):
    """The health-ratio gate beside the per-format tolerance."""
    bound = health_bound(lane_depth(fmt, K))
    assert res["max_err"] <= bound, (f"{tag}: max_err {res['max_err']:.3e} above the health bound {bound:.3e} "
                                     f"(ratio {res['max_err'] / (bound / 4.0):.1f}) at {res['argmax']}")


def log(msg):
    print(f"[gpu-test] {msg}", flush=True)


def dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def run_fused(w, x, act, m=None, r=None, out_shape=None, inplace=False, stream=None):
    """Runs gemv_fused on device copies; returns the float32 output (host) and
    the device tensors used."""
    Wd = dev(w.data)
    xd = dev(np.asarray(x, dtype=np.float32))
    shape = tuple(out_shape) if out_shape else (w.N,)
    md = dev(np.asarray(m, dtype=np.float32).reshape(shape)) if m is not None else None
    rd = dev(np.asarray(r, dtype=np.float32).reshape(shape)) if r is not None else None
    if inplace:
        dst = rd if act == "add" else md
    else:
        dst = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    binding.gemv_fused(Wd, w.fmt, w.N, w.K, xd, act, mul_operand=md, add_operand=rd, dst=dst)
    torch.cuda.synchronize()
    return host(dst).reshape(-1).copy(), dict(W=Wd, x=xd, m=md, r=rd, dst=dst)


def check_parity(w, x, act, m=None, r=None, out_shape=None, inplace=False, tag=""):
    log(f"parity {tag} fmt={w.fmt} N={w.N} K={w.K} act={act} inplace={inplace}")
    g, _ = run_fused(w, x, act, m=m, r=r, out_shape=out_shape, inplace=inplace)
    y, acc, absacc = oracle.reference(w.fmt, w.N, w.K, w.data, x, act, m=m, r=r)
    mm = None if m is None else np.asarray(m, dtype=np.float32).reshape(-1)
    rr = None if r is None else np.asarray(r, dtype=np.float32).reshape(-1)
    res = compare(g, y, acc, absacc, act, m=mm, r=rr)
    tol = TOLERANCE[w.fmt]
    assert np.all(np.isfinite(g)), f"{tag}: non-finite output"
    assert res["max_err"] <= tol, f"{tag}: max_err {res['max_err']:.3e} > {tol} at {res['argmax']} ({res})"
    assert_healthy(res, w.fmt, w.K, tag)
    return g, y, res


def run_ncols(w, X, act, M=None, R=None, out_shape=None, inplace=False):
    B = X.shape[0]
    shape = tuple(out_shape) if out_shape else (B, w.N)
    Wd, Xd = dev(w.data), dev(X)
    Md = dev(M.reshape(shape)) if M is not None else None
    Rd = dev(R.reshape(shape)) if R is not None else None
    if inplace:
        dst = Rd if act == "add" else Md
    else:
        dst = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    binding.gemv_fused_ncols(Wd, w.fmt, w.N, w.K, B, Xd, act, mul_operand=Md, add_operand=Rd, dst=dst)
    torch.cuda.synchronize()
    return host(dst).reshape(-1).copy()


def check_ncols(w, X, act, M=None, R=None, out_shape=None, inplace=False, tag=""):
    log(f"ncols {tag} fmt={w.fmt} N={w.N} K={w.K} ncols={X.shape[0]} act={act} inplace={inplace}")
    g = run_ncols(w, X, act, M, R, out_shape, inplace)
    Y, acc, absacc = oracle.ncols_reference(w.fmt, w.N, w.K, w.data, X, act, M=M, R=R)
    res = compare(g, Y.reshape(-1), acc.reshape(-1), absacc.reshape(-1), act,
                  m=None if M is None else M.reshape(-1), r=None if R is None else R.reshape(-1))
    assert np.all(np.isfinite(g)), tag
    assert res["max_err"] <= TOLERANCE[w.fmt], f"{tag}: {res}"
    # the matrix-core kernel carries x as two 16-bit pieces (2^-20 relative);
    # the gate applies to the vector-ALU kernels, which keep x in float32
    if binding.gemv_ncols_kernel(w.fmt, w.N, w.K, X.shape[0]) != "columns_matrix":
        assert_healthy(res, w.fmt, w.K, tag)
    return g
