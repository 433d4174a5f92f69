"""Helpers for the GPU tests: device copies, one fused call, the oracle beside it."""
import numpy as np
import torch

import oracle
from oracle.compare import TOLERANCE, compare
from decode_gemv_elementwise_amd import binding


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
    return g, y, res
