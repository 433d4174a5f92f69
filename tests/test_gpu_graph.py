"""Every entry point captured into a HIP graph and replayed gives the same bits
as the eager call.  The benchmark times the kernels as graph replays, so this
is what makes its figures figures of the same computation.  Each graph is
replayed three times, with the program's own eager work (a fill of the output,
a synchronisation) between replays, and every replay is compared with the
eager result.  No kernel here clears memory with a memset node; outputs are
written whole by each launch."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from decode_gemv_elementwise_amd import binding, synth
from gpu_util import dev, host, log

pytestmark = pytest.mark.gpu


def _replays_match(tag, launch, out):
    """launch(dst) enqueues one call writing dst on the current stream."""
    eager = torch.full_like(out, float("nan"))
    launch(eager)
    torch.cuda.synchronize()
    want = host(eager).copy()
    assert np.all(np.isfinite(want)), tag
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            launch(out)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = host(out)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"{tag}: replay {rep} differs"
    del g


ONE_COLUMN = [("f16", 4096, 4096, "add"), ("bf16", 14336, 4096, "silu_mul"), ("f32", 33, 257, "sigmoid"),
              ("q8b32", 4096, 14336, "mul"), ("q4b32", 14336, 4096, "silu"), ("q4b32", 4096, 14336, "add")]


@pytest.mark.parametrize("fmt,N,K,act", ONE_COLUMN)
def test_graph_one_column(fmt, N, K, act):
    log(f"graph gemv_fused {fmt} {N}x{K} {act}")
    rng = np.random.default_rng(40)
    w = synth.random_weights(rng, fmt, N, K)
    Wd, xd = dev(w.data), dev(synth.draw_vec(rng, K))
    op = dev(synth.draw_vec(rng, N))
    kw = {"add_operand": op} if act == "add" else ({"mul_operand": op} if act in ("mul", "silu_mul") else {})
    out = torch.empty(N, dtype=torch.float32, device="cuda")
    _replays_match(f"{fmt} {N}x{K} {act}", lambda d: binding.gemv_fused(Wd, fmt, N, K, xd, act, dst=d, **kw), out)


def test_graph_epilogue_and_glu():
    log("graph gemv_epilogue, gemv_glu")
    rng = np.random.default_rng(41)
    N, K = 14336, 4096
    acc, m = dev(synth.draw_vec(rng, N)), dev(synth.draw_vec(rng, N))
    out = torch.empty(N, dtype=torch.float32, device="cuda")
    _replays_match("epilogue silu_mul", lambda d: binding.gemv_epilogue("silu_mul", N, acc, mul_operand=m, dst=d), out)
    wg = synth.random_weights(rng, "q4b32", N, K)
    wu = synth.random_weights(rng, "q4b32", N, K)
    Wg, Wu, xd = dev(wg.data), dev(wu.data), dev(synth.draw_vec(rng, K))
    _replays_match("glu q4", lambda d: binding.gemv_glu(Wg, Wu, "q4b32", N, K, xd, "silu", dst=d), out)


NCOLS = [("f16", 4096, 4096, 8, "add"), ("q4b32", 14336, 4096, 4, "silu"), ("q4b32", 4096, 14336, 8, "add"),
         ("f32", 1024, 1024, 3, "mul"), ("bf16", 64, 257, 2, "none")]


@pytest.mark.parametrize("fmt,N,K,B,act", NCOLS)
def test_graph_ncols(fmt, N, K, B, act):
    log(f"graph gemv_fused_ncols {fmt} {N}x{K} ncols={B} {act} kernel={binding.gemv_ncols_kernel(fmt, N, K, B)}")
    rng = np.random.default_rng(42)
    w = synth.random_weights(rng, fmt, N, K)
    Wd = dev(w.data)
    X = dev(np.stack([synth.draw_vec(rng, K) for _ in range(B)]))
    op = dev(np.stack([synth.draw_vec(rng, N) for _ in range(B)]))
    kw = {"add_operand": op} if act == "add" else ({"mul_operand": op} if act in ("mul", "silu_mul") else {})
    out = torch.empty(B, N, dtype=torch.float32, device="cuda")
    _replays_match(f"ncols {fmt} {B}", lambda d: binding.gemv_fused_ncols(Wd, fmt, N, K, B, X, act, dst=d, **kw), out)


@pytest.mark.parametrize("fmt,B", [("f16", 4), ("q4b32", 4)])
def test_graph_glu_ncols(fmt, B):
    log(f"graph gemv_glu_ncols {fmt} ncols={B}")
    rng = np.random.default_rng(44)
    N, K = 14336, 4096
    wg = synth.random_weights(rng, fmt, N, K)
    wu = synth.random_weights(rng, fmt, N, K)
    Wg, Wu = dev(wg.data), dev(wu.data)
    X = dev(np.stack([synth.draw_vec(rng, K) for _ in range(B)]))
    out = torch.empty(B, N, dtype=torch.float32, device="cuda")
    _replays_match(f"glu ncols {fmt}", lambda d: binding.gemv_glu_ncols(Wg, Wu, fmt, N, K, B, X, "silu", dst=d), out)


def test_graph_hadamard():
    log("graph gemv_fwht_signed, gemv_fused_fwht")
    rng = np.random.default_rng(43)
    N, K = 4096, 4096
    x = dev(synth.draw_vec(rng, 2 * K))
    signs = dev(np.where(rng.random(K) < 0.5, -1.0, 1.0).astype(np.float32))
    out = torch.empty(2 * K, dtype=torch.float32, device="cuda")
    _replays_match("fwht", lambda d: binding.gemv_fwht_signed(x, signs, 2, K, 1024, K, d), out)
    w = synth.random_weights(rng, "f16", N, K)
    Wd, r = dev(w.data), dev(synth.draw_vec(rng, N))
    out = torch.empty(N, dtype=torch.float32, device="cuda")
    _replays_match("fused fwht", lambda d: binding.gemv_fused_fwht(Wd, "f16", N, K, x[:K], signs, 1024, K, "add",
                                                                   add_operand=r, dst=d), out)
