"""GPU parity of the signed Hadamard transform (gemv_fwht_signed) and of the
product after it in one launch (gemv_fused_fwht) against the oracle, and the
bit-for-bit agreement of the fused call with the two-call composition."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from oracle.compare import FWHT_TOLERANCE, TOLERANCE, compare
from decode_gemv_elementwise_amd import binding, synth
from gpu_util import dev, host, log

pytestmark = pytest.mark.gpu


def _signs(rng, ns):
    return rng.choice([-1.0, 1.0], size=ns).astype(np.float32)


def run_fwht(x, s, n, inplace=False, x_offset=0):
    """x: [nrows, K] float32 on the host.  x_offset > 0 places x (and dst) at
    a 4-byte, not 16-byte, aligned address."""
    nrows, K = x.shape
    buf = torch.zeros(nrows * K + x_offset, dtype=torch.float32, device="cuda")
    buf[x_offset:] = dev(x.reshape(-1))
    xd = buf[x_offset:]
    sd = dev(s)
    if inplace:
        dst = xd
    else:
        dbuf = torch.full((nrows * K + x_offset,), float("nan"), dtype=torch.float32, device="cuda")
        dst = dbuf[x_offset:]
    binding.gemv_fwht_signed(xd, sd, nrows, K, n, s.size, dst)
    torch.cuda.synchronize()
    return host(dst).reshape(nrows, K).copy()


def check_fwht(x, s, n, tag, **kw):
    log(f"fwht {tag} rows={x.shape[0]} K={x.shape[1]} n={n} nsigns={s.size} {kw}")
    g = run_fwht(x, s, n, **kw)
    y, d = oracle.fwht_signed(x, s, n)
    diff = np.abs(g.astype(np.float64) - y)
    err = np.where(diff == 0, 0.0, diff / np.maximum(np.abs(y), d))
    assert np.all(np.isfinite(g)), tag
    assert err.max() <= FWHT_TOLERANCE, f"{tag}: max err {err.max():.3e}"
    return g


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024])
def test_fwht_block_sizes(n):
    rng = np.random.default_rng(n)
    K = 4096
    x = rng.normal(size=(2, K)).astype(np.float32)
    check_fwht(x, _signs(rng, K), n, "block")


@pytest.mark.parametrize("nrows,K,n,ns", [(1, 5120, 1024, 5120), (3, 1024, 1024, 1024), (1, 14336, 1024, 1024),
                                          (5, 96, 32, 3), (1, 7, 1, 7), (2, 6, 2, 1), (1, 1032, 8, 4),
                                          (4, 3072, 512, 6)])
def test_fwht_shapes_and_sign_periods(nrows, K, n, ns):
    rng = np.random.default_rng(K + n + ns)
    x = rng.normal(size=(nrows, K)).astype(np.float32)
    check_fwht(x, _signs(rng, ns), n, f"K={K}")


def test_fwht_in_place_and_unaligned():
    rng = np.random.default_rng(3)
    x = rng.normal(size=(2, 4096)).astype(np.float32)
    s = _signs(rng, 4096)
    a = check_fwht(x, s, 1024, "out of place")
    b = check_fwht(x, s, 1024, "in place", inplace=True)
    c = check_fwht(x, s, 1024, "unaligned", x_offset=1)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))


def test_fwht_unit_vectors_and_involution():
    """e_j gives column j of H / sqrt(n) exactly for n = 4^k (the scale is a
    power of two); applying the unsigned transform again gives back x * s."""
    n = 256
    x = np.zeros((4, n), np.float32)
    js = [0, 1, 77, 255]
    for r, j in enumerate(js):
        x[r, j] = 1.0
    g = run_fwht(x, np.ones(1, np.float32), n)
    for r, j in enumerate(js):
        want = np.array([(-1.0) ** bin(i & j).count("1") for i in range(n)], np.float32) / 16.0
        assert np.array_equal(g[r], want), j
    rng = np.random.default_rng(4)
    x = rng.normal(size=(1, 2048)).astype(np.float32)
    s = _signs(rng, 2048)
    y = run_fwht(run_fwht(x, s, 1024), np.ones(1, np.float32), 1024)
    assert np.max(np.abs(y - x * s)) <= 1e-5 * np.max(np.abs(x))


def test_fwht_deterministic():
    rng = np.random.default_rng(5)
    x = rng.normal(size=(3, 5120)).astype(np.float32)
    s = _signs(rng, 5120)
    a = run_fwht(x, s, 1024)
    b = run_fwht(x, s, 1024)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ------------------------------------------------------------------ the product after the transform

def run_fused_fwht(w, x, s, n, act, m=None, r=None, out_shape=None, inplace=False):
    Wd, xd, sd = dev(w.data), dev(x), dev(s)
    shape = tuple(out_shape) if out_shape else (w.N,)
    md = dev(m.reshape(shape)) if m is not None else None
    rd = dev(r.reshape(shape)) if r is not None else None
    if inplace:
        dst = rd if act == "add" else md
    else:
        dst = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    binding.gemv_fused_fwht(Wd, w.fmt, w.N, w.K, xd, sd, n, s.size, act, mul_operand=md, add_operand=rd, dst=dst)
    torch.cuda.synchronize()
    return host(dst).reshape(-1).copy()


def check_fused_fwht(w, x, s, n, act, m=None, r=None, tag="", **kw):
    log(f"fused fwht {tag} fmt={w.fmt} N={w.N} K={w.K} n={n} nsigns={s.size} act={act}")
    g = run_fused_fwht(w, x, s, n, act, m, r, **kw)
    y, acc, absacc = oracle.fwht_gemv_reference(w.fmt, w.N, w.K, w.data, x, s, n, act, m=m, r=r)
    res = compare(g, y, acc, absacc, act, m=m, r=r)
    assert np.all(np.isfinite(g)), tag
    assert res["max_err"] <= TOLERANCE[w.fmt], f"{tag}: {res}"
    return g


@pytest.mark.parametrize("fmt", synth.FORMATS)
@pytest.mark.parametrize("N,K,n", [(1, 1024, 1024), (300, 4096, 1024), (67, 14336, 1024), (1003, 5120, 1024),
                                   (33, 4096, 64), (17, 2048, 2)])
def test_fused_fwht_parity(fmt, N, K, n):
    rng = np.random.default_rng(N + K + n)
    w = synth.random_weights(rng, fmt, N, K)
    x = rng.normal(size=K).astype(np.float32)
    r = rng.normal(size=N).astype(np.float32)
    check_fused_fwht(w, x, _signs(rng, K), n, "add", r=r, tag="parity")


@pytest.mark.parametrize("fmt", synth.FORMATS)
@pytest.mark.parametrize("act", list(synth.ACTS))
def test_fused_fwht_equals_transform_then_gemv_bitwise(fmt, act):
    rng = np.random.default_rng(len(act) * 10 + synth.FORMATS.index(fmt))
    N, K, n = 515, 4096, 1024
    w = synth.random_weights(rng, fmt, N, K)
    x = rng.normal(size=K).astype(np.float32)
    s = _signs(rng, 1024)
    m = rng.normal(size=N).astype(np.float32) if act in ("silu_mul", "mul") else None
    r = rng.normal(size=N).astype(np.float32) if act == "add" else None
    g = check_fused_fwht(w, x, s, n, act, m, r, tag="vs composition")
    xp = dev(run_fwht(x.reshape(1, K), s, n).reshape(-1))
    dst = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    binding.gemv_fused(dev(w.data), fmt, N, K, xp, act, mul_operand=None if m is None else dev(m),
                       add_operand=None if r is None else dev(r), dst=dst)
    torch.cuda.synchronize()
    assert np.array_equal(g.view(np.uint32), host(dst).view(np.uint32))


def test_fused_fwht_in_place_view_add():
    rng = np.random.default_rng(6)
    w = synth.random_weights(rng, "q8b32", 4096, 6144)
    x = rng.normal(size=6144).astype(np.float32)
    r = rng.normal(size=4096).astype(np.float32)
    check_fused_fwht(w, x, _signs(rng, 6144), 1024, "add", r=r, out_shape=(32, 128), inplace=True, tag="view")


def test_fused_fwht_identity_weights_give_the_transform():
    """W = I (f32): the product returns the transformed x itself."""
    rng = np.random.default_rng(7)
    K = 2048
    eye = synth.Weights("f32", K, K, np.eye(K, dtype=np.float32).view(np.uint8).reshape(-1))
    x = rng.normal(size=K).astype(np.float32)
    s = _signs(rng, K)
    g = run_fused_fwht(eye, x, s, 1024, "none")
    t = run_fwht(x.reshape(1, K), s, 1024).reshape(-1)
    assert np.array_equal(g.view(np.uint32), t.view(np.uint32))


def test_fused_fwht_rejects_generic_path_shapes():
    rng = np.random.default_rng(8)
    w = synth.random_weights(rng, "f16", 8, 4100)
    dst = torch.full((8,), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(binding.GemvError) as e:
        binding.gemv_fused_fwht(dev(w.data), "f16", 8, 4100, dev(rng.normal(size=4100).astype(np.float32)),
                                dev(np.ones(4, np.float32)), 4, 4, "none", dst=dst)
    assert e.value.status == binding.STATUS_CODE["GEMV_E_DIM"]
    torch.cuda.synchronize()
    assert torch.all(dst == 7.0)


def _signs_then_nan(s):
    """The signs on the device followed by NaN: a read past the last sign
    would turn a transformed value into NaN."""
    buf = torch.full((s.size + 64,), float("nan"), dtype=torch.float32, device="cuda")
    buf[: s.size] = dev(s)
    return buf


@pytest.mark.parametrize("nrows,K,n", [(1, 256, 256), (2, 1536, 512), (1, 1040, 16), (3, 48, 16)])
def test_fwht_sign_reads_stay_in_bounds(nrows, K, n):
    """K not a multiple of the 1024-value tile, with nsigns = K or n (a
    multiple of 16, the aligned 16-sign path): lanes past the end of the row
    must not read past the sign vector."""
    rng = np.random.default_rng(K + n)
    for ns in sorted({K, n}):
        x = rng.normal(size=(nrows, K)).astype(np.float32)
        s = _signs(rng, ns)
        log(f"fwht bounds rows={nrows} K={K} n={n} nsigns={ns}")
        xd = dev(x.reshape(-1))
        dst = torch.full((nrows * K,), float("nan"), dtype=torch.float32, device="cuda")
        binding.gemv_fwht_signed(xd, _signs_then_nan(s), nrows, K, n, ns, dst)
        torch.cuda.synchronize()
        g = host(dst).reshape(nrows, K)
        y, d = oracle.fwht_signed(x, s, n)
        assert np.all(np.isfinite(g))
        diff = np.abs(g.astype(np.float64) - y)
        assert np.max(np.where(diff == 0, 0.0, diff / np.maximum(np.abs(y), d))) <= FWHT_TOLERANCE


@pytest.mark.parametrize("fmt", synth.FORMATS)
@pytest.mark.parametrize("N,K,n", [(37, 1536, 512), (5, 256, 256)])
def test_fused_fwht_sign_reads_stay_in_bounds(fmt, N, K, n):
    rng = np.random.default_rng(N + K)
    w = synth.random_weights(rng, fmt, N, K)
    x = rng.normal(size=K).astype(np.float32)
    r = rng.normal(size=N).astype(np.float32)
    for ns in sorted({K, n}):
        s = _signs(rng, ns)
        log(f"fused fwht bounds fmt={fmt} N={N} K={K} n={n} nsigns={ns}")
        dst = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
        binding.gemv_fused_fwht(dev(w.data), fmt, N, K, dev(x), _signs_then_nan(s), n, ns, "add",
                                add_operand=dev(r), dst=dst)
        torch.cuda.synchronize()
        g = host(dst)
        y, acc, absacc = oracle.fwht_gemv_reference(fmt, N, K, w.data, x, s, n, "add", r=r)
        assert np.all(np.isfinite(g))
        assert compare(g, y, acc, absacc, "add", r=r)["max_err"] <= TOLERANCE[fmt]
