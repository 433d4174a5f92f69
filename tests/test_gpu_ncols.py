"""GPU parity of gemv_fused_ncols (2..8 destination columns over one W)
against the oracle.  f32 and bf16 columns (vector-ALU column kernel) also
equal one gemv_fused call per column bit for bit; f16 and the block formats
run on the matrix cores where the shape fits, and there every column is
independent of its position among the others, bit for bit."""
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from oracle.compare import TOLERANCE, compare
from decode_gemv_elementwise_amd import binding, synth
from gpu_util import check_ncols, dev, host, log, run_ncols

pytestmark = pytest.mark.gpu

ALL_ACTS = list(synth.ACTS)


def _operands(rng, act, B, N):
    M = rng.normal(size=(B, N)).astype(np.float32) if act in ("silu_mul", "mul") else None
    R = rng.normal(size=(B, N)).astype(np.float32) if act == "add" else None
    return M, R


SHAPES = [(1, 64), (33, 96), (300, 4096), (1003, 2048), (67, 14336), (17, 4128)]


@pytest.mark.parametrize("fmt", synth.FORMATS)
@pytest.mark.parametrize("ncols", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("N,K", SHAPES)
def test_ncols_parity(fmt, ncols, N, K):
    rng = np.random.default_rng(N * 7 + K + 1000 * ncols)
    w = synth.random_weights(rng, fmt, N, K)
    X = rng.normal(size=(ncols, K)).astype(np.float32)
    check_ncols(w, X, "none", tag=f"{N}x{K}")


@pytest.mark.parametrize("fmt", synth.FORMATS)
@pytest.mark.parametrize("act", ALL_ACTS)
def test_ncols_epilogues(fmt, act):
    rng = np.random.default_rng(zlib.crc32(f"{fmt}/{act}".encode()))
    N, K, B = 515, 1024, 3
    w = synth.random_weights(rng, fmt, N, K)
    X = rng.normal(size=(B, K)).astype(np.float32)
    M, R = _operands(rng, act, B, N)
    check_ncols(w, X, act, M, R, tag="epilogue")


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("N,K", [(5, 7), (64, 1001), (130, 4099)])
def test_ncols_unaligned_k(fmt, N, K):
    """Rows that are not whole 16-byte chunks take the element-wise kernel."""
    rng = np.random.default_rng(N + K)
    w = synth.random_weights(rng, fmt, N, K)
    X = rng.normal(size=(5, K)).astype(np.float32)
    check_ncols(w, X, "silu", tag="unaligned")


def _one_column(w, x, act, m, r):
    Wd, xd = dev(w.data), dev(x)
    md = dev(m) if m is not None else None
    rd = dev(r) if r is not None else None
    dst = torch.full((w.N,), float("nan"), dtype=torch.float32, device="cuda")
    binding.gemv_fused(Wd, w.fmt, w.N, w.K, xd, act, mul_operand=md, add_operand=rd, dst=dst)
    torch.cuda.synchronize()
    return host(dst).copy()


@pytest.mark.parametrize("fmt", synth.FORMATS)
@pytest.mark.parametrize("N,K,act", [(300, 4096, "silu_mul"), (67, 14336, "add"), (17, 4128, "sigmoid"),
                                     (40, 96, "mul")])
def test_ncols_columns_equal_one_column_calls_bitwise(fmt, N, K, act):
    """On the vector-ALU column kernel (f32 at 8 columns, every format at 2)."""
    rng = np.random.default_rng(N + K + 77)
    w = synth.random_weights(rng, fmt, N, K)
    B = 8 if fmt == "f32" else 2
    assert binding.gemv_ncols_kernel(fmt, N, K, B) != "columns_matrix"
    X = rng.normal(size=(B, K)).astype(np.float32)
    M, R = _operands(rng, act, B, N)
    log(f"ncols-vs-one-column fmt={fmt} N={N} K={K} act={act}")
    g = run_ncols(w, X, act, M, R).reshape(B, N)
    for b in range(B):
        one = _one_column(w, X[b], act, None if M is None else M[b], None if R is None else R[b])
        assert np.array_equal(g[b].view(np.uint32), one.view(np.uint32)), (fmt, b)


@pytest.mark.parametrize("fmt", synth.FORMATS)
@pytest.mark.parametrize("N,K,B,act", [(300, 4096, 8, "silu_mul"), (67, 14336, 3, "add"), (17, 4128, 5, "sigmoid"),
                                       (40, 96, 2, "mul"), (5000, 1024, 4, "add"), (4100, 2048, 7, "silu")])
def test_ncols_columns_independent_of_position_bitwise(fmt, N, K, B, act):
    """Rolling the columns of x (and of the operands) rolls the result
    columns, bit for bit, on every path."""
    rng = np.random.default_rng(N + K + 99)
    w = synth.random_weights(rng, fmt, N, K)
    X = rng.normal(size=(B, K)).astype(np.float32)
    M, R = _operands(rng, act, B, N)
    log(f"ncols position fmt={fmt} N={N} K={K} B={B} act={act}")
    g = check_ncols(w, X, act, M, R, tag="position").reshape(B, N)
    for sft in range(1, B):
        roll = lambda a: None if a is None else np.roll(a, -sft, axis=0)
        g2 = run_ncols(w, roll(X), act, roll(M), roll(R)).reshape(B, N)
        assert np.array_equal(g2.view(np.uint32), np.roll(g, -sft, axis=0).view(np.uint32)), (fmt, sft)


def test_ncols_odd_k_columns_equal_one_column_calls_bitwise():
    rng = np.random.default_rng(5)
    w = synth.random_weights(rng, "f32", 70, 1001)
    X = rng.normal(size=(4, 1001)).astype(np.float32)
    g = run_ncols(w, X, "silu").reshape(4, 70)
    for b in range(4):
        assert np.array_equal(g[b].view(np.uint32), _one_column(w, X[b], "silu", None, None).view(np.uint32))


def test_ncols_one_is_gemv_fused():
    rng = np.random.default_rng(6)
    w = synth.random_weights(rng, "q4b32", 257, 4096)
    x = rng.normal(size=(1, 4096)).astype(np.float32)
    g = run_ncols(w, x, "silu")
    assert np.array_equal(g.view(np.uint32), _one_column(w, x[0], "silu", None, None).view(np.uint32))


def test_ncols_inplace_and_view():
    rng = np.random.default_rng(7)
    w = synth.random_weights(rng, "q8b32", 4096, 6144)
    B = 4
    X = rng.normal(size=(B, 6144)).astype(np.float32)
    R = rng.normal(size=(B, 4096)).astype(np.float32)
    check_ncols(w, X, "add", R=R, out_shape=(B, 32, 128), tag="view")
    check_ncols(w, X, "add", R=R, out_shape=(B, 32, 128), inplace=True, tag="view in place")
    M = rng.normal(size=(B, 4096)).astype(np.float32)
    check_ncols(w, X, "silu_mul", M=M, inplace=True, tag="silu_mul in place")


@pytest.mark.parametrize("fmt,N,K,act", [("bf16", 16 * 600 + 7, 4096, "add"), ("f16", 16 * 600 + 7, 4096, "silu_mul"),
                                         ("f32", 16 * 600 + 7, 2048, "sigmoid"), ("q8b32", 16 * 700 + 9, 4096, "mul"),
                                         ("q4b32", 16 * 700 + 9, 4096, "silu")])
def test_ncols_resident_grid_walks_ragged_tiles(fmt, N, K, act):
    """Two columns with more 16-row tiles than resident workgroups and a
    ragged last tile: the one-shot form's workgroups walk several tiles
    each; every column must match the oracle and the one-column call bit
    for bit."""
    B = 2
    assert binding.gemv_ncols_kernel(fmt, N, K, B) == "columns"
    rng = np.random.default_rng(zlib.crc32(f"ncolsresident/{fmt}/{N}/{K}".encode()))
    w = synth.random_weights(rng, fmt, N, K)
    X = rng.normal(size=(B, K)).astype(np.float32)
    M, R = _operands(rng, act, B, N)
    log(f"ncols resident grid fmt={fmt} N={N} K={K} act={act}")
    g = check_ncols(w, X, act, M, R, tag="resident grid").reshape(B, N)
    for b in range(B):
        one = _one_column(w, X[b], act, None if M is None else M[b], None if R is None else R[b])
        assert np.array_equal(g[b].view(np.uint32), one.view(np.uint32)), (fmt, b)


@pytest.mark.parametrize("fmt,N,K,act", [("q4b32", 14336, 4096, "silu"), ("bf16", 14336, 4096, "silu_mul"),
                                         ("f16", 4096, 4096, "add"), ("q4b32", 4096, 14336, "add"),
                                         ("q8b32", 14336, 4096, "mul"), ("q8b32", 4096, 6144, "silu"),
                                         ("bf16", 4096, 14336, "add")])
def test_ncols_full_size(fmt, N, K, act):
    rng = np.random.default_rng(8)
    w = synth.random_weights(rng, fmt, N, K)
    B = 8
    X = rng.normal(size=(B, K)).astype(np.float32)
    M, R = _operands(rng, act, B, N)
    check_ncols(w, X, act, M, R, tag="full size")


def test_ncols_zero_and_identity():
    rng = np.random.default_rng(9)
    N = K = 256
    X = rng.normal(size=(6, K)).astype(np.float32)
    zero = synth.Weights("f16", N, K, np.zeros(N * K, dtype=np.float16).view(np.uint8))
    g = run_ncols(zero, X, "sigmoid")
    assert np.all(g == 0.5)
    eye = synth.Weights("f32", N, K, np.eye(N, K, dtype=np.float32).view(np.uint8).reshape(-1))
    g = run_ncols(eye, X, "none")
    assert np.array_equal(g, X.reshape(-1))


def test_ncols_rejected_call_writes_nothing():
    rng = np.random.default_rng(10)
    w = synth.random_weights(rng, "f16", 64, 64)
    Wd = dev(w.data)
    Xd = dev(rng.normal(size=(9, 64)).astype(np.float32))
    dst = torch.full((9, 64), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(binding.GemvError) as e:
        binding.gemv_fused_ncols(Wd, "f16", 64, 64, 9, Xd, "none", dst=dst)
    assert e.value.status == binding.STATUS_CODE["GEMV_E_DIM"]
    torch.cuda.synchronize()
    assert torch.all(dst == 7.0)


@pytest.mark.parametrize("fmt", ["f32", "bf16", "f16", "q4b32"])
def test_ncols_x_not_16_byte_aligned(fmt):
    """x at a 4-byte (not 16-byte) aligned address: the result equals the
    same call with 16-byte aligned x bit for bit, and on the vector-ALU
    kernel (f32 here) the one-column calls too."""
    rng = np.random.default_rng(11)
    N, K, B = 200, 2048, 6
    w = synth.random_weights(rng, fmt, N, K)
    X = rng.normal(size=(B, K)).astype(np.float32)
    Wd = dev(w.data)
    buf = torch.zeros(B * K + 1, dtype=torch.float32, device="cuda")
    buf[1:] = dev(X.reshape(-1))
    xv = buf[1:]
    assert xv.data_ptr() % 16 == 4
    dst = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    log(f"ncols unaligned x fmt={fmt}")
    binding.gemv_fused_ncols(Wd, fmt, N, K, B, xv, "silu", dst=dst)
    torch.cuda.synchronize()
    g = host(dst)
    Y, acc, absacc = oracle.ncols_reference(fmt, N, K, w.data, X, "silu")
    res = compare(g.reshape(-1), Y.reshape(-1), acc.reshape(-1), absacc.reshape(-1), "silu")
    assert res["max_err"] <= TOLERANCE[fmt], res
    aligned = run_ncols(w, X, "silu").reshape(B, N)
    assert np.array_equal(g.view(np.uint32), aligned.view(np.uint32))
    if binding.gemv_ncols_kernel(fmt, N, K, B) != "columns_matrix":
        for b in range(B):
            one = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
            binding.gemv_fused(Wd, fmt, N, K, xv[b * K:(b + 1) * K], "silu", dst=one)
            torch.cuda.synchronize()
            assert np.array_equal(g[b].view(np.uint32), host(one).view(np.uint32)), b


@pytest.mark.parametrize("fmt", ["f16", "bf16", "q8b32", "q4b32"])
@pytest.mark.parametrize("N,K", [(300, 4096), (4500, 1024)])
def test_ncols_wide_range_columns(fmt, N, K):
    """Columns far apart in magnitude (each column takes its own power-of-two
    scale on the matrix-core path), a zero column, a column with one large
    value among tiny ones, a subnormal column: each within tolerance, the
    zero column exactly epilogue(0)."""
    rng = np.random.default_rng(N + K + 12)
    w = synth.random_weights(rng, fmt, N, K)
    X = rng.normal(size=(6, K)).astype(np.float32)
    X[0] *= np.float32(1e30)
    X[1] *= np.float32(1e-30)
    X[2] = 0.0
    X[3] *= np.float32(1e-4)
    X[3, K // 3] = 1e4
    X[4] = (X[4] * np.float32(1e-40)).astype(np.float32)
    X[5] *= np.float32(3e4)
    g = check_ncols(w, X, "add", R=rng.normal(size=(6, N)).astype(np.float32), tag="wide range").reshape(6, N)
    g0 = check_ncols(w, X, "sigmoid", tag="wide range sigmoid").reshape(6, N)
    assert np.all(g0[2] == 0.5)


@pytest.mark.parametrize("fmt,N,K,ncols,kernel", [
    ("f16", 4096, 4096, 8, "columns_matrix"), ("f16", 300, 4096, 5, "columns_matrix"),
    ("f16", 4096, 4096, 4, "columns"), ("f16", 14336, 4096, 8, "columns"),
    ("q4b32", 14336, 4096, 4, "columns_matrix"), ("q4b32", 14336, 4096, 8, "columns_matrix"),
    ("q4b32", 300, 4096, 8, "columns_matrix"), ("q4b32", 4100, 2048, 7, "columns_matrix"),
    ("q4b32", 4096, 4096, 2, "columns"), ("q4b32", 4096, 14336, 8, "columns_matrix"), ("q4b32", 33, 96, 8, "columns"),
    ("q4b32", 67, 14336, 6, "columns_matrix"), ("f16", 4096, 14336, 8, "columns_matrix"), ("f16", 4096, 14336, 6, "columns"),
    ("q8b32", 4096, 6144, 4, "columns_matrix"), ("q8b32", 14336, 4096, 8, "columns_matrix"),
    ("q8b32", 4096, 6144, 8, "columns_matrix"), ("q8b32", 4096, 4096, 4, "columns"), ("q8b32", 4096, 14336, 3, "columns"),
    ("bf16", 4096, 4096, 8, "columns_matrix"), ("bf16", 4096, 4096, 4, "columns"), ("bf16", 14336, 4096, 8, "columns"),
    ("bf16", 4096, 2048, 6, "columns"), ("bf16", 4096, 2048, 8, "columns_matrix"),
    ("f32", 4096, 4096, 8, "columns"), ("f32", 64, 1001, 4, "columns_generic"), ("f16", 64, 64, 1, "one_column")])
def test_ncols_kernel_choice(fmt, N, K, ncols, kernel):
    """The shapes the tests above rely on to reach each kernel take it."""
    assert binding.gemv_ncols_kernel(fmt, N, K, ncols) == kernel


MATRIX_SHAPES = [("f16", 300, 4096, 8), ("bf16", 300, 4096, 6), ("q4b32", 300, 4096, 7), ("q8b32", 4096, 6144, 4),
                 ("q4b32", 67, 14336, 8), ("f16", 67, 14336, 7), ("q8b32", 4096, 6144, 8)]


@pytest.mark.parametrize("fmt,N,K,B", MATRIX_SHAPES)
@pytest.mark.parametrize("act", ALL_ACTS)
def test_ncols_matrix_core_epilogues(fmt, N, K, B, act):
    """Every epilogue on the matrix-core kernels (single segment and
    segmented, as the kernel query confirms)."""
    assert binding.gemv_ncols_kernel(fmt, N, K, B) == "columns_matrix"
    rng = np.random.default_rng(zlib.crc32(f"mx/{fmt}/{N}/{K}/{act}".encode()))
    w = synth.random_weights(rng, fmt, N, K)
    X = rng.normal(size=(B, K)).astype(np.float32)
    M, R = _operands(rng, act, B, N)
    check_ncols(w, X, act, M, R, tag=f"matrix {act}")


@pytest.mark.parametrize("fmt,N,K,B", [("q4b32", 14336 + 37, 4096, 4), ("q4b32", 8192 + 5, 2048, 6),
                                       ("q8b32", 14336 + 21, 4096, 6), ("q4b32", 4096 + 3, 14336, 3),
                                       ("f16", 4096 - 9, 4096, 6)])
def test_ncols_matrix_core_ragged_rows(fmt, N, K, B):
    """Row counts that leave the last 16-row tile (and the last workgroup of
    2 or 4 tiles) partly empty."""
    assert binding.gemv_ncols_kernel(fmt, N, K, B) == "columns_matrix"
    rng = np.random.default_rng(N + K + B)
    w = synth.random_weights(rng, fmt, N, K)
    X = rng.normal(size=(B, K)).astype(np.float32)
    R = rng.normal(size=(B, N)).astype(np.float32)
    check_ncols(w, X, "add", R=R, tag="ragged")
