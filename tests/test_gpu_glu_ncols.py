"""The gated pair over several destination columns (gemv_glu_ncols) against
the oracle, and against the one-column pair bit for bit: column b is
act(W_gate x_b) * (W_up x_b), each row sum formed in the one-column order."""
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from oracle.compare import TOLERANCE, compare_glu
from decode_gemv_elementwise_amd import binding, synth
from gpu_util import assert_healthy, dev, host, log

pytestmark = pytest.mark.gpu

SHAPES = [(1, 32), (33, 96), (300, 512), (1003, 4096), (67, 14336), (17, 4128)]


def _run(wg, wu, X, act, out_shape=None):
    B = X.shape[0]
    Wg, Wu, Xd = dev(wg.data), dev(wu.data), dev(X)
    dst = torch.full(out_shape or (B, wg.N), float("nan"), dtype=torch.float32, device="cuda")
    binding.gemv_glu_ncols(Wg, Wu, wg.fmt, wg.N, wg.K, B, Xd, act, dst=dst)
    torch.cuda.synchronize()
    return host(dst).reshape(B, wg.N)


def _one(wg, wu, x, act):
    dst = torch.full((wg.N,), float("nan"), dtype=torch.float32, device="cuda")
    binding.gemv_glu(dev(wg.data), dev(wu.data), wg.fmt, wg.N, wg.K, dev(x), act, dst=dst)
    torch.cuda.synchronize()
    return host(dst)


def _check(wg, wu, X, act, tag):
    log(f"glu ncols {tag} fmt={wg.fmt} N={wg.N} K={wg.K} ncols={X.shape[0]} act={act}")
    G = _run(wg, wu, X, act)
    Y, g, gA, u, uA = oracle.glu_ncols_reference(wg.fmt, wg.N, wg.K, wg.data, wu.data, X, act)
    res = compare_glu(G.reshape(-1), Y.reshape(-1), act, g.reshape(-1), gA.reshape(-1), u.reshape(-1),
                      uA.reshape(-1))
    assert np.all(np.isfinite(G)), tag
    assert res["max_err"] <= TOLERANCE[wg.fmt], f"{tag}: {res}"
    # silu over columns the matrix cores take runs there (x as two 16-bit
    # pieces); every other route keeps x in float32 on the vector ALUs
    if act != "silu" or binding.gemv_ncols_kernel(wg.fmt, wg.N, wg.K, X.shape[0]) != "columns_matrix":
        assert_healthy(res, wg.fmt, wg.K, tag)
    return G


@pytest.mark.parametrize("fmt", synth.FORMATS)
@pytest.mark.parametrize("N,K", SHAPES)
def test_glu_ncols_parity(fmt, N, K):
    rng = np.random.default_rng(zlib.crc32(f"gluncols/{fmt}/{N}/{K}".encode()))
    wg = synth.random_weights(rng, fmt, N, K)
    wu = synth.random_weights(rng, fmt, N, K)
    for B, act in ((2, "silu"), (5, "sigmoid"), (8, "silu")):
        X = np.stack([synth.draw_vec(rng, K) for _ in range(B)])
        _check(wg, wu, X, act, f"{fmt} {N}x{K} {B} {act}")


@pytest.mark.parametrize("fmt", synth.FORMATS)
@pytest.mark.parametrize("N,K,B", [(300, 4096, 3), (67, 14336, 8), (17, 4128, 2), (1003, 512, 6)])
def test_glu_ncols_columns_equal_one_column_pair_bitwise(fmt, N, K, B):
    log(f"glu ncols == gemv_glu per column, {fmt} {N}x{K} ncols={B}")
    rng = np.random.default_rng(zlib.crc32(f"glubit/{fmt}/{N}/{K}".encode()))
    wg = synth.random_weights(rng, fmt, N, K)
    wu = synth.random_weights(rng, fmt, N, K)
    X = np.stack([synth.draw_vec(rng, K) for _ in range(B)])
    # sigmoid always takes the one-launch pair; silu too unless the matrix
    # cores take the columns (then two matrix-core launches, not bitwise)
    acts = ["sigmoid"] + (["silu"] if binding.gemv_ncols_kernel(fmt, N, K, B) != "columns_matrix" else [])
    for act in acts:
        G = _run(wg, wu, X, act)
        for b in range(B):
            assert np.array_equal(G[b].view(np.uint32), _one(wg, wu, X[b], act).view(np.uint32)), (fmt, act, b)


@pytest.mark.parametrize("fmt,N,K,B", [("q4b32", 14336, 4096, 4), ("q4b32", 4096, 4096, 8), ("q8b32", 14336, 4096, 8)])
def test_glu_ncols_matrix_core_route(fmt, N, K, B):
    """Where the columns run on the matrix cores, silu pairs take two
    matrix-core launches (up into dst, gate with silu * up in place); the
    result still meets the oracle, and equals that composition by hand."""
    assert binding.gemv_ncols_kernel(fmt, N, K, B) == "columns_matrix"
    rng = np.random.default_rng(zlib.crc32(f"glumfma/{fmt}/{N}/{K}/{B}".encode()))
    wg = synth.random_weights(rng, fmt, N, K)
    wu = synth.random_weights(rng, fmt, N, K)
    X = np.stack([synth.draw_vec(rng, K) for _ in range(B)])
    G = _check(wg, wu, X, "silu", f"{fmt} {N}x{K} {B} matrix-core route")
    Wg, Wu, Xd = dev(wg.data), dev(wu.data), dev(X)
    up = torch.empty(B, N, dtype=torch.float32, device="cuda")
    out = torch.empty(B, N, dtype=torch.float32, device="cuda")
    binding.gemv_fused_ncols(Wu, fmt, N, K, B, Xd, "none", dst=up)
    binding.gemv_fused_ncols(Wg, fmt, N, K, B, Xd, "silu_mul", mul_operand=up, dst=out)
    torch.cuda.synchronize()
    assert np.array_equal(G.view(np.uint32), host(out).view(np.uint32))
    _check(wg, wu, X, "sigmoid", f"{fmt} {N}x{K} {B} sigmoid, one launch")


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_glu_ncols_odd_k_generic_path(fmt):
    log(f"glu ncols odd K {fmt}")
    rng = np.random.default_rng(71)
    wg = synth.random_weights(rng, fmt, 40, 1001)
    wu = synth.random_weights(rng, fmt, 40, 1001)
    X = np.stack([synth.draw_vec(rng, 1001) for _ in range(4)])
    G = _check(wg, wu, X, "silu", f"{fmt} odd K")
    for b in range(4):
        assert np.array_equal(G[b].view(np.uint32), _one(wg, wu, X[b], "silu").view(np.uint32)), (fmt, b)


@pytest.mark.parametrize("fmt,N,K,B", [("bf16", 8 * 600 + 5, 4096, 4), ("q8b32", 8 * 700 + 3, 4096, 2),
                                       ("q4b32", 8 * 700 + 3, 4096, 2)])
def test_glu_ncols_resident_grid_walks_ragged_tiles(fmt, N, K, B):
    """Shapes with more 8-row tiles than resident workgroups and a ragged last
    tile: the one-shot pair's workgroups walk several tiles each, and every
    column must still match the oracle and the one-column pair bit for bit."""
    assert binding.gemv_ncols_kernel(fmt, N, K, B) == "columns"
    rng = np.random.default_rng(zlib.crc32(f"gluresident/{fmt}/{N}/{K}/{B}".encode()))
    wg = synth.random_weights(rng, fmt, N, K)
    wu = synth.random_weights(rng, fmt, N, K)
    X = np.stack([synth.draw_vec(rng, K) for _ in range(B)])
    for act in ("silu", "sigmoid"):
        G = _check(wg, wu, X, act, f"resident grid {fmt} {N}x{K} {B} {act}")
        for b in range(B):
            assert np.array_equal(G[b].view(np.uint32), _one(wg, wu, X[b], act).view(np.uint32)), (fmt, act, b)


def test_glu_ncols_full_size_gate_up():
    """The 4-bit gate and up projections of the decode layer, 4 columns."""
    rng = np.random.default_rng(72)
    wl = synth.q4b32_decode_layer(0)
    wg, wu = wl.weights["Wgate"], wl.weights["Wup"]
    X = np.stack([synth.draw_vec(rng, wg.K) for _ in range(4)])
    _check(wg, wu, X, "silu", "q4 14336x4096 gate/up")


def test_glu_ncols_one_column_and_rejections():
    log("glu ncols: one column, rejected calls")
    rng = np.random.default_rng(73)
    wg = synth.random_weights(rng, "bf16", 64, 256)
    wu = synth.random_weights(rng, "bf16", 64, 256)
    X = synth.draw_vec(rng, 256)[None, :]
    assert np.array_equal(_run(wg, wu, X, "sigmoid")[0].view(np.uint32),
                          _one(wg, wu, X[0], "sigmoid").view(np.uint32))
    Wg, Wu, Xd = dev(wg.data), dev(wu.data), dev(np.stack([X[0]] * 3))
    dst = torch.full((3, 64), 7.0, dtype=torch.float32, device="cuda")
    for act, nc, status in (("add", 3, "GEMV_E_ACT"), ("silu", 9, "GEMV_E_DIM"), ("silu", 2, "GEMV_E_DIM")):
        with pytest.raises(binding.GemvError) as e:
            binding.gemv_glu_ncols(Wg, Wu, "bf16", 64, 256, nc, Xd, act, dst=dst)
        assert e.value.status == binding.STATUS_CODE[status]
    torch.cuda.synchronize()
    assert torch.all(dst == 7.0)
