"""Special values on the one-column path, pinned by IEEE arithmetic: the
oracle evaluates the same products and sums in double, so a NaN weight (or a
NaN block scale) must poison exactly its row, and an infinite x_j must give
NaN in every row whose weight at j is exactly zero (0 * inf) and an infinity
of the weight's sign in every other row.  The epilogues then map +inf, -inf
and NaN accumulators as the oracle's do (sigmoid: 1, 0, NaN; silu: +inf, NaN,
NaN).  The same holds over several destination columns, on the vector-ALU
column kernels and on the matrix-core ones (whose x pieces carry an infinity
whole and scale each column by its largest finite magnitude), for the gated
pair on each of its routes, and through the signed Hadamard prologue."""
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from oracle.compare import TOLERANCE, compare, compare_glu
from decode_gemv_elementwise_amd import binding, synth
from gpu_util import host, log, run_fused, run_ncols

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


# (format, N, K, columns, kernel the call takes): the matrix-core kernels in
# one segment and segmented, and the vector-ALU column kernels
COLUMN_SHAPES = [
    ("f16", 300, 4096, 8, "columns_matrix"), ("bf16", 300, 4096, 6, "columns_matrix"),
    ("q4b32", 300, 4096, 7, "columns_matrix"), ("q8b32", 4096, 6144, 4, "columns_matrix"),
    ("q4b32", 67, 14336, 8, "columns_matrix"), ("f16", 67, 14336, 7, "columns_matrix"),
    ("f16", 4096, 4096, 4, "columns"), ("bf16", 4096, 4096, 4, "columns"), ("q8b32", 4096, 4096, 4, "columns"),
    ("q4b32", 4096, 4096, 2, "columns"), ("q4b32", 33, 96, 8, "columns"), ("f32", 4096, 4096, 8, "columns"),
]


def _finite_columns_within_tolerance(w, X, act, g, Y, acc, absacc, R, cols, tag):
    for b in cols:
        res = compare(g[b], Y[b], acc[b], absacc[b], act, r=None if R is None else R[b])
        assert res["max_err"] <= TOLERANCE[w.fmt], f"{tag} column {b}: {res}"


@pytest.mark.parametrize("fmt,N,K,B,kernel", COLUMN_SHAPES)
def test_columns_infinite_and_nan_x_follow_ieee(fmt, N, K, B, kernel):
    """Column 0 holds +inf at position j, column 1 -inf there beside a large
    finite value, column 2 a NaN, column 3 +inf and -inf side by side; W is
    zero at (row, j) for three rows.  Every column's NaN / infinity pattern
    and signs match the oracle's IEEE double arithmetic, and the remaining
    (finite) columns are unaffected."""
    assert binding.gemv_ncols_kernel(fmt, N, K, B) == kernel
    log(f"special: columns {fmt} {N}x{K} ncols={B} ({kernel})")
    rng = np.random.default_rng(zlib.crc32(f"special-cols/{fmt}/{N}/{K}/{B}".encode()))
    w = synth.random_weights(rng, fmt, N, K)
    j = K // 3 - 5
    zero_rows = [i for i in (3, 17, 40) if i < N]
    for i in zero_rows:
        _set_weight(w, i, j, "zero")
    X = synth.draw_vec(rng, B * K).reshape(B, K)
    X[0, j] = np.inf
    X[1, j] = -np.inf
    X[1, j + 7] = 1e30
    if B > 2:
        X[2, j + 1] = np.nan
    if B > 3:
        X[3, j] = np.inf
        X[3, j + 2] = -np.inf
    R = synth.draw_vec(rng, B * N).reshape(B, N)
    g = run_ncols(w, X, "add", R=R).reshape(B, N)
    Y, acc, absacc = oracle.ncols_reference(fmt, N, K, w.data, X, "add", R=R)
    Y = np.asarray(Y)
    for i in zero_rows:
        assert np.isnan(Y[0, i]) and np.isnan(Y[1, i])
    for b in range(min(B, 4)):
        _same_pattern(g[b], Y[b], f"{fmt} {kernel} column {b}")
    _finite_columns_within_tolerance(w, X, "add", g, Y, acc, absacc, R, range(4, B), f"{fmt} {kernel}")


@pytest.mark.parametrize("fmt,N,K,B,kernel", COLUMN_SHAPES)
def test_columns_nan_weight_poisons_only_its_row(fmt, N, K, B, kernel):
    """A NaN weight (a NaN block scale for the block formats) makes its row
    NaN in every column and leaves every other row as the oracle has it."""
    assert binding.gemv_ncols_kernel(fmt, N, K, B) == kernel
    log(f"special: columns NaN weight {fmt} {N}x{K} ncols={B} ({kernel})")
    rng = np.random.default_rng(zlib.crc32(f"special-cols-w/{fmt}/{N}/{K}/{B}".encode()))
    w = synth.random_weights(rng, fmt, N, K)
    _set_weight(w, 5, 37, "nan")
    X = synth.draw_vec(rng, B * K).reshape(B, K)
    g = run_ncols(w, X, "silu").reshape(B, N)
    Y, acc, absacc = oracle.ncols_reference(fmt, N, K, w.data, X, "silu")
    Y = np.asarray(Y)
    assert np.isnan(g[:, 5]).all() and np.isnan(Y[:, 5]).all()
    rest = np.arange(N) != 5
    assert np.isfinite(g[:, rest]).all() and np.isfinite(Y[:, rest]).all()
    for b in range(B):
        res = compare(g[b, rest], Y[b, rest], acc[b, rest], absacc[b, rest], "silu")
        assert res["max_err"] <= TOLERANCE[fmt], f"{fmt} {kernel} column {b}: {res}"


def _run_glu(wg, wu, X, act):
    """gemv_glu (X of one row) or gemv_glu_ncols; the float32 output [B, N]."""
    B = X.shape[0]
    Wg, Wu = torch.from_numpy(wg.data).cuda(), torch.from_numpy(wu.data).cuda()
    Xd = torch.from_numpy(np.ascontiguousarray(X.reshape(-1) if B == 1 else X)).cuda()
    dst = torch.full((B, wg.N) if B > 1 else (wg.N,), float("nan"), dtype=torch.float32, device="cuda")
    if B == 1:
        binding.gemv_glu(Wg, Wu, wg.fmt, wg.N, wg.K, Xd, act, dst=dst)
    else:
        binding.gemv_glu_ncols(Wg, Wu, wg.fmt, wg.N, wg.K, B, Xd, act, dst=dst)
    torch.cuda.synchronize()
    return host(dst).reshape(B, wg.N)


# (format, N, K, columns): one column, the one-launch pair over columns, and
# (silu on a shape whose columns run on the matrix cores) the two matrix-core
# launches
GLU_SHAPES = [("q4b32", 256, 4096, 1), ("bf16", 256, 4096, 1), ("q4b32", 4096, 4096, 2), ("f16", 300, 4096, 8),
              ("q8b32", 4096, 6144, 4)]


@pytest.mark.parametrize("fmt,N,K,B", GLU_SHAPES)
@pytest.mark.parametrize("act", ["silu", "sigmoid"])
def test_gated_pair_special_values_follow_ieee(fmt, N, K, B, act):
    """The gated pair with +inf (column 0), -inf (column 1) and NaN (column
    2) in x and zero gate or up weights at the infinite position in a few
    rows: NaN / infinity patterns and signs as in the oracle's act(g) * u."""
    log(f"special: gated pair {fmt} {N}x{K} ncols={B} {act}")
    rng = np.random.default_rng(zlib.crc32(f"special-glu/{fmt}/{N}/{K}/{B}/{act}".encode()))
    wg = synth.random_weights(rng, fmt, N, K)
    wu = synth.random_weights(rng, fmt, N, K)
    j = K // 2 + 3
    for i in (2, 9):
        _set_weight(wg, i, j, "zero")
    for i in (9, 30):
        _set_weight(wu, i, j, "zero")
    X = synth.draw_vec(rng, B * K).reshape(B, K)
    X[0, j] = np.inf
    if B > 1:
        X[1, j] = -np.inf
    if B > 2:
        X[2, j + 1] = np.nan
    g = _run_glu(wg, wu, X, act)
    for b in range(B):
        Y, G, AG, U, AU = (np.asarray(a) for a in oracle.glu_reference(fmt, N, K, wg.data, wu.data, X[b], act))
        if b < 3:  # a special value in this column: every row is +-inf or NaN
            _same_pattern(g[b], Y, f"{fmt} {act} column {b}")
            assert not np.isfinite(Y).any()
        else:      # the other columns are untouched
            res = compare_glu(g[b], Y, act, G, AG, U, AU)
            assert res["max_err"] <= TOLERANCE[fmt], f"{fmt} {act} column {b}: {res}"


@pytest.mark.parametrize("fmt", ["f16", "q4b32"])
def test_hadamard_prologue_special_values_follow_ieee(fmt):
    """An infinite x through the fused signed transform: its 1024-block
    becomes infinities of the transform's signs (one infinity meets only
    finite values in the butterflies), then the product; a NaN x poisons its
    block.  NaN / infinity patterns and signs as in the oracle."""
    log(f"special: signed FWHT prologue {fmt}")
    N, K, n = 96, 2048, 1024
    rng = np.random.default_rng(zlib.crc32(f"special-fwht/{fmt}".encode()))
    w = synth.random_weights(rng, fmt, N, K)
    s = np.where(rng.random(K) < 0.5, -1.0, 1.0).astype(np.float32)
    for x_special in (np.inf, np.nan):
        x = synth.draw_vec(rng, K)
        x[300] = x_special
        r = synth.draw_vec(rng, N)
        dst = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
        binding.gemv_fused_fwht(torch.from_numpy(w.data).cuda(), fmt, N, K, torch.from_numpy(x).cuda(),
                                torch.from_numpy(s).cuda(), n, K, "add", add_operand=torch.from_numpy(r).cuda(), dst=dst)
        torch.cuda.synchronize()
        g = host(dst)
        y = np.asarray(oracle.fwht_gemv_reference(fmt, N, K, w.data, x, s, n, "add", r=r)[0])
        _same_pattern(g, y, f"{fmt} FWHT x={x_special}")
        assert not np.isfinite(y).any()
