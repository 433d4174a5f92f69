"""Special values on the one-column path, pinned by IEEE arithmetic: the
oracle evaluates the same products and sums in double, so a NaN weight (or a
NaN block scale) must poison exactly its row, and an infinite x_j must give
NaN in every row whose weight at j is exactly zero (0 * inf) and an infinity
of the weight's sign in every other row.  The epilogues then map +inf, -inf
and NaN accumulators as the oracle's do (sigmoid: 1, 0, NaN; silu: +inf, NaN,
NaN).  The matrix-core column kernels are not covered: they scale each column
of x by a power of two taken from its largest magnitude, which an infinite or
NaN x leaves undefined."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from decode_gemv_elementwise_amd import synth
from gpu_util import host, log, run_fused

pytestmark = pytest.mark.gpu

N, K = 64, 256


def _a256(v):
    return (v + 255) // 256 * 256


def _scales_view(w):
    off = _a256(w.N * w.K) if w.fmt == "q8b32" else _a256(w.N * w.K // 2)
    return w.data[off:off + 2 * w.N * (w.K // 32)].view(np.uint16).reshape(w.N, w.K // 32)


def _set_weight(w, i, j, kind):
    """Plants a NaN (kind 'nan') or an exact zero (kind 'zero') at W[i, j]; for
    the block formats a NaN goes into the block's fp16 scale."""
    if w.fmt == "f32":
        w.data.view(np.float32).reshape(w.N, w.K)[i, j] = np.nan if kind == "nan" else 0.0
    elif w.fmt in ("f16", "bf16"):
        nan = 0x7E00 if w.fmt == "f16" else 0x7FC0
        w.data[:2 * w.N * w.K].view(np.uint16).reshape(w.N, w.K)[i, j] = nan if kind == "nan" else 0
    elif kind == "nan":
        _scales_view(w)[i, j // 32] = 0x7E00
    elif w.fmt == "q8b32":
        w.data[i * w.K + j] = 0
    else:  # code 8 encodes zero
        b = (i * w.K + j) // 2
        w.data[b] = (w.data[b] & 0xF0) | 8 if j % 2 == 0 else (w.data[b] & 0x0F) | 0x80


def _same_pattern(g, y, tag):
    assert np.array_equal(np.isnan(g), np.isnan(y)), f"{tag}: NaN rows {np.flatnonzero(np.isnan(g))} vs {np.flatnonzero(np.isnan(y))}"
    inf = np.isinf(y)
    assert np.array_equal(np.isinf(g), inf), f"{tag}: infinite rows differ"
    assert np.array_equal(np.sign(g[inf]), np.sign(y[inf])), f"{tag}: signs of infinities differ"


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_nan_weight_poisons_only_its_row(fmt):
    log(f"special: NaN weight {fmt}")
    rng = np.random.default_rng(50)
    w = synth.random_weights(rng, fmt, N, K)
    _set_weight(w, 5, 37, "nan")
    x = synth.draw_vec(rng, K)
    g, _ = run_fused(w, x, "none")
    y, _, _ = oracle.reference(fmt, N, K, w.data, x, "none")
    assert np.isnan(g[5]) and np.isnan(y[5])
    rest = np.arange(N) != 5
    assert np.all(np.isfinite(g[rest])) and np.all(np.isfinite(y[rest]))
    scale = np.maximum(np.abs(y[rest]), 1e-3)
    assert np.max(np.abs(g[rest] - y[rest]) / scale) < 1e-2


@pytest.mark.parametrize("fmt", synth.FORMATS)
@pytest.mark.parametrize("act", ["none", "sigmoid", "silu", "silu_mul", "add"])
def test_infinite_x_follows_ieee(fmt, act):
    log(f"special: infinite x {fmt} {act}")
    rng = np.random.default_rng(51)
    w = synth.random_weights(rng, fmt, N, K)
    j = 100
    for i in (3, 17, 40):
        _set_weight(w, i, j, "zero")
    x = synth.draw_vec(rng, K)
    x[j] = np.inf
    m = synth.draw_vec(rng, N) if act == "silu_mul" else None
    r = synth.draw_vec(rng, N) if act == "add" else None
    g, _ = run_fused(w, x, act, m=m, r=r)
    y, _, _ = oracle.reference(fmt, N, K, w.data, x, act, m=m, r=r)
    y = np.asarray(y)
    assert np.isnan(y[[3, 17, 40]]).all()
    _same_pattern(g, y, f"{fmt} {act}")
    fin = np.isfinite(y)
    if fin.any():  # sigmoid of -inf is 0, of +inf is 1: exact
        assert np.array_equal(g[fin], y[fin].astype(np.float32)), f"{fmt} {act}"
