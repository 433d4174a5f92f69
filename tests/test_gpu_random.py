"""Seeded random shapes against the oracle: every format, ragged N, odd K for
the float formats, K a multiple of 32 for the block formats, every epilogue,
in place or not, one column and 2..8 columns.  The list holds a few large
cases so that the matrix-core column kernels (single and segmented) and the
long-row one-column paths are drawn too.  Each case logs its parameters
before it runs; the cases are fixed by the seed, so a failure is
reproducible on the CPU side of the test."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from decode_gemv_elementwise_amd import binding, synth
from gpu_util import check_ncols, check_parity, log

pytestmark = pytest.mark.gpu

ACTS = list(synth.ACTS)


def _shape(rng, fmt, big):
    if big:
        N = int(rng.choice([2048, 4096, 6144, 8192])) + int(rng.integers(0, 40))
        K = int(rng.choice([2048, 4096, 6144, 8192, 14336]))
        return N, K
    N = int(rng.integers(1, 3000))
    if fmt in ("q8b32", "q4b32"):
        K = 32 * int(rng.integers(1, 200))
    else:
        K = int(rng.integers(1, 9000))
    return N, K


def _cases(seed, n, ncols):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = synth.FORMATS[int(rng.integers(0, len(synth.FORMATS)))]
        big = i % 3 == 2
        N, K = _shape(rng, fmt, big)
        B = int(rng.integers(2, 9)) if ncols else 1
        act = ACTS[int(rng.integers(0, len(ACTS)))]
        inplace = act in ("add", "mul", "silu_mul") and bool(rng.integers(0, 2))
        out.append((i, fmt, N, K, B, act, inplace))
    return out


@pytest.mark.parametrize("case", _cases(1234, 40, ncols=False), ids=lambda c: f"{c[1]}-{c[2]}x{c[3]}-{c[5]}")
def test_random_one_column(case):
    i, fmt, N, K, _, act, inplace = case
    rng = np.random.default_rng(5000 + i)
    w = synth.random_weights(rng, fmt, N, K)
    x = synth.draw_vec(rng, K)
    m = synth.draw_vec(rng, N) if act in ("mul", "silu_mul") else None
    r = synth.draw_vec(rng, N) if act == "add" else None
    check_parity(w, x, act, m=m, r=r, inplace=inplace, tag=f"random #{i}")


@pytest.mark.parametrize("case", _cases(4321, 40, ncols=True), ids=lambda c: f"{c[1]}-{c[2]}x{c[3]}-b{c[4]}-{c[5]}")
def test_random_ncols(case):
    i, fmt, N, K, B, act, inplace = case
    log(f"random ncols #{i}: kernel {binding.gemv_ncols_kernel(fmt, N, K, B)}")
    rng = np.random.default_rng(6000 + i)
    w = synth.random_weights(rng, fmt, N, K)
    X = np.stack([synth.draw_vec(rng, K) for _ in range(B)])
    M = np.stack([synth.draw_vec(rng, N) for _ in range(B)]) if act in ("mul", "silu_mul") else None
    R = np.stack([synth.draw_vec(rng, N) for _ in range(B)]) if act == "add" else None
    check_ncols(w, X, act, M=M, R=R, inplace=inplace, tag=f"random ncols #{i}")
