"""Pins for the CPU oracle: each check ties it to something other than itself
(library conversions, hand-built byte images, exact rational arithmetic,
closed forms, textbook identities), chosen so that a plausible mistake
(a dropped term, a wrong sign, index or nibble order, a transposed operand,
a wrong plane offset) fails at least one of them."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle.compare import TOLERANCE, compare, error_scale, glu_error_scale, health_bound
from decode_gemv_elementwise_amd import synth

U = 2.0 ** -53


def gamma(n):
    return n * U / (1 - n * U)


# ----------------------------------------------------------------- decoders

def test_f16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode("f16", 1, 65536, bits.view(np.uint8))[0]
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signed zeros keep their sign
    assert math.copysign(1.0, got[0x8000]) == -1.0


def test_bf16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode("bf16", 1, 65536, bits.view(np.uint8))[0]
    want = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_f32_decode_matches_numpy():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=4096, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = np.where(np.isnan(f), np.float32(1.5), f).astype(np.float32)
    got = oracle.decode("f32", 4, 1024, f.view(np.uint8)).reshape(-1)
    assert np.array_equal(got, f.astype(np.float64))


def _image(fixture):
    buf = np.zeros(fixture["nbytes"], dtype=np.uint8)
    for off, hx in fixture["segments"]:
        b = np.frombuffer(bytes.fromhex(hx), dtype=np.uint8)
        buf[off:off + b.size] = b
    return buf


@pytest.mark.parametrize("fmt", ["q4b32", "q8b32"])
def test_block_decode_golden(golden_dir, fmt):
    fx = json.load(open(os.path.join(golden_dir, f"{fmt}_blocks.json")))
    N, K = fx["N"], fx["K"]
    assert oracle.weight_bytes(fmt, N, K) == fx["nbytes"]
    got = oracle.decode(fmt, N, K, _image(fx))
    for n, key in enumerate(["expected_row0", "expected_row1"]):
        want = [Fraction(s) for s in fx[key]]
        assert [Fraction(v) for v in got[n]] == want, (fmt, n)


def test_weight_bytes_spec():
    assert oracle.weight_bytes("f32", 256, 256) == 262144
    assert oracle.weight_bytes("f16", 4096, 4096) == 33554432
    assert oracle.weight_bytes("bf16", 14336, 4096) == 117440512
    assert oracle.weight_bytes("q8b32", 4096, 6144) == 26738688   # 25165824 codes + 1572864 scales
    assert oracle.weight_bytes("q4b32", 4096, 14336) == 33030144  # 29360128 nibbles + 3670016 scales
    assert oracle.weight_bytes("q4b32", 3, 32) == 256 + 6         # 48 code bytes padded to 256
    assert oracle.weight_bytes("q8b32", 3, 32) == 256 + 6
    assert oracle.weight_bytes("q4b32", 4, 33) == -1
    assert oracle.weight_bytes("f32", 0, 4) == -1
    assert oracle.weight_bytes("f16", 4, 0) == -1


@pytest.mark.parametrize("fmt", ["q4b32", "q8b32"])
def test_pack_decode_roundtrip(fmt):
    """Packed codes + scales decode to code * scale exactly (code - 8 for 4-bit),
    with the scale read by numpy's binary16 conversion."""
    rng = np.random.default_rng(7)
    N, K = 5, 96
    w = synth.random_weights(rng, fmt, N, K)
    got = oracle.decode(fmt, N, K, w.data)
    codes = w.codes.astype(np.float64) - (8.0 if fmt == "q4b32" else 0.0)
    want = codes * np.repeat(w.scales.astype(np.float64), 32, axis=1)
    assert np.array_equal(got, want)
    assert w.data.size == oracle.weight_bytes(fmt, N, K)


# ----------------------------------------------------------------- GEMV

def _exact_values(w: synth.Weights):
    """Exact weight values as Fractions, decoded independently of the oracle."""
    N, K = w.N, w.K
    if w.fmt == "f32":
        v = w.data.view(np.float32).reshape(N, K).astype(np.float64)
    elif w.fmt == "f16":
        v = w.data.view(np.float16).reshape(N, K).astype(np.float64)
    elif w.fmt == "bf16":
        t = torch.from_numpy(w.data.view(np.int16).copy()).view(torch.bfloat16)
        v = t.to(torch.float64).numpy().reshape(N, K)
    else:
        off = 8 if w.fmt == "q4b32" else 0
        return [[Fraction(int(w.codes[i, j]) - off) * Fraction(float(w.scales[i, j // 32]))
                 for j in range(K)] for i in range(N)]
    return [[Fraction(float(v[i, j])) for j in range(K)] for i in range(N)]


@pytest.mark.parametrize("fmt,N,K", [("f32", 1, 1), ("f32", 3, 7), ("f32", 6, 16), ("f16", 4, 13),
                                     ("bf16", 5, 11), ("q8b32", 3, 32), ("q8b32", 2, 64),
                                     ("q4b32", 4, 32), ("q4b32", 3, 64)])
def test_gemv_brute_force_exact(fmt, N, K):
    """Against exact rational arithmetic: |acc - exact| <= gamma_{K-1} A and the
    same for A itself (recursive summation bound)."""
    rng = np.random.default_rng(N * 1000 + K)
    w = synth.random_weights(rng, fmt, N, K)
    x = synth.draw_vec(rng, K)
    acc, absacc = oracle.gemv(fmt, N, K, w.data, x)
    ex = _exact_values(w)
    xf = [Fraction(float(v)) for v in x]
    for i in range(N):
        exact = sum(ex[i][j] * xf[j] for j in range(K))
        A = sum(abs(ex[i][j] * xf[j]) for j in range(K))
        bound = gamma(max(K - 1, 0)) * float(A)
        assert abs(float(Fraction(acc[i]) - exact)) <= bound * (1 + 1e-12) + 1e-300
        assert abs(float(Fraction(absacc[i]) - A)) <= bound * (1 + 1e-12) + 1e-300
        # all products are exact in double, so fsum gives the correctly rounded sum
        prods = [float(ex[i][j] * xf[j]) for j in range(K)]
        assert abs(acc[i] - math.fsum(prods)) <= bound * (1 + 1e-12) + 1e-300


def test_gemv_integer_exact():
    """8-bit blocks with scale 1 and small integer x: every partial sum is an
    integer below 2^24, so the result is exact and unique."""
    rng = np.random.default_rng(3)
    N, K = 8, 6144
    codes = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    scales = np.ones((N, K // 32), dtype=np.float16)
    w = synth.pack_q8b32(codes, scales)
    xi = rng.integers(-3, 4, size=K)
    acc, absacc = oracle.gemv("q8b32", N, K, w, xi.astype(np.float32))
    want = codes.astype(np.int64) @ xi
    wantA = np.abs(codes.astype(np.int64)) @ np.abs(xi)
    assert np.array_equal(acc, want.astype(np.float64))
    assert np.array_equal(absacc, wantA.astype(np.float64))


def test_gemv_zero_weights():
    N, K = 7, 33
    x = synth.draw_vec(np.random.default_rng(0), K)
    acc, absacc = oracle.gemv("f32", N, K, np.zeros(N * K, dtype=np.float32).view(np.uint8), x)
    assert np.all(acc == 0) and np.all(absacc == 0)


def test_gemv_identity_q4():
    """4-bit identity: code 9 (value +1 at scale 1) on the diagonal, code 8 (value 0) elsewhere."""
    N = K = 64
    codes = np.full((N, K), 8, dtype=np.uint8)
    np.fill_diagonal(codes, 9)
    w = synth.pack_q4b32(codes, np.ones((N, K // 32), dtype=np.float16))
    x = synth.draw_vec(np.random.default_rng(5), K)
    acc, _ = oracle.gemv("q4b32", N, K, w, x)
    assert np.array_equal(acc, x.astype(np.float64))


def test_gemv_permutation_f16():
    N = K = 40
    perm = np.random.default_rng(11).permutation(K)
    W = np.zeros((N, K), dtype=np.float16)
    W[np.arange(N), perm] = 1.0
    x = synth.draw_vec(np.random.default_rng(12), K)
    acc, _ = oracle.gemv("f16", N, K, W.view(np.uint8), x)
    assert np.array_equal(acc, x[perm].astype(np.float64))


def test_gemv_rank1_nonsquare():
    """W = u v^T with dyadic entries (every sum exact): acc = u (v . x).  N != K
    so a transposed operand cannot pass."""
    rng = np.random.default_rng(13)
    N, K = 5, 12
    u = rng.choice([-2.0, -1.0, -0.5, 0.5, 1.0, 2.0], size=N)
    v = rng.choice([-1.0, -0.25, 0.25, 0.5, 1.0, 3.0], size=K)
    x = rng.choice([-2.0, -1.0, 0.0, 1.0, 4.0], size=K).astype(np.float32)
    W = np.outer(u, v).astype(np.float32)
    acc, _ = oracle.gemv("f32", N, K, W.view(np.uint8), x)
    assert np.array_equal(acc, u * float(v @ x.astype(np.float64)))


def test_gemv_row_slices_match_full():
    rng = np.random.default_rng(17)
    w = synth.random_weights(rng, "q4b32", 50, 64)
    x = synth.draw_vec(rng, 64)
    acc, absacc = oracle.gemv("q4b32", 50, 64, w.data, x)
    a2, b2 = oracle.gemv("q4b32", 50, 64, w.data, x, rows=(13, 29))
    assert np.array_equal(acc[13:29], a2) and np.array_equal(absacc[13:29], b2)


# ----------------------------------------------------------------- epilogues

def test_epilogue_closed_forms():
    ln3 = math.log(3.0)
    assert oracle.sigmoid(ln3) == pytest.approx(0.75, rel=4e-16)
    assert oracle.sigmoid(-ln3) == pytest.approx(0.25, rel=4e-16)
    assert oracle.silu(ln3) == pytest.approx(0.75 * ln3, rel=4e-16)
    assert oracle.sigmoid(0.0) == 0.5
    assert oracle.silu(0.0) == 0.0
    assert oracle.sigmoid(-800.0) == 0.0 and oracle.sigmoid(800.0) == 1.0


def test_epilogue_against_library_logistic():
    a = np.random.default_rng(19).normal(0, 4, size=2000)
    s = scipy.special.expit(a)
    y_sig = oracle.epilogue("sigmoid", a)
    y_silu = oracle.epilogue("silu", a)
    assert np.allclose(y_sig, s, rtol=4e-16, atol=0)
    assert np.allclose(y_silu, a * s, rtol=6e-16, atol=0)
    # identities: sigma(a) + sigma(-a) = 1, silu(a) - silu(-a) = a
    assert np.allclose(y_sig + oracle.epilogue("sigmoid", -a), 1.0, rtol=0, atol=4e-16)
    assert np.allclose(y_silu - oracle.epilogue("silu", -a), a, rtol=1e-15, atol=1e-300)


def test_epilogue_operands():
    rng = np.random.default_rng(23)
    a = rng.normal(size=300)
    m = synth.draw_vec(rng, 300)
    r = synth.draw_vec(rng, 300)
    s = scipy.special.expit(a)
    assert np.allclose(oracle.epilogue("silu_mul", a, m=m), a * s * m.astype(np.float64), rtol=1e-15, atol=0)
    assert np.array_equal(oracle.epilogue("mul", a, m=m), a * m.astype(np.float64))
    assert np.array_equal(oracle.epilogue("add", a, r=r), a + r.astype(np.float64))
    ones = np.ones(300, dtype=np.float32)
    zeros = np.zeros(300, dtype=np.float32)
    assert np.array_equal(oracle.epilogue("silu_mul", a, m=ones), oracle.epilogue("silu", a))
    assert np.array_equal(oracle.epilogue("mul", a, m=ones), oracle.epilogue("none", a))
    assert np.array_equal(oracle.epilogue("add", a, r=zeros), oracle.epilogue("none", a))
    with pytest.raises(ValueError):
        oracle.epilogue("add", a)
    with pytest.raises(ValueError):
        oracle.epilogue("mul", a)


def test_zero_w_epilogues():
    N, K = 16, 32
    x = synth.draw_vec(np.random.default_rng(29), K)
    m = synth.draw_vec(np.random.default_rng(30), N)
    r = synth.draw_vec(np.random.default_rng(31), N)
    w = np.zeros(N * K, dtype=np.float16).view(np.uint8)
    want = {"none": 0.0, "sigmoid": 0.5, "silu": 0.0, "silu_mul": 0.0, "mul": 0.0}
    for act, v in want.items():
        y, _, _ = oracle.reference("f16", N, K, w, x, act, m=m, r=r)
        assert np.all(y == v), act
    y, _, _ = oracle.reference("f16", N, K, w, x, "add", r=r)
    assert np.array_equal(y, r.astype(np.float64))


def test_identity_w_epilogues():
    """Identity W gives epilogue(x), with the logistic taken from scipy."""
    N = K = 64
    codes = np.full((N, K), 8, dtype=np.uint8)
    np.fill_diagonal(codes, 9)
    w = synth.pack_q4b32(codes, np.ones((N, K // 32), dtype=np.float16))
    rng = np.random.default_rng(37)
    x = synth.draw_vec(rng, K)
    m = synth.draw_vec(rng, N)
    xd = x.astype(np.float64)
    s = scipy.special.expit(xd)
    y, _, _ = oracle.reference("q4b32", N, K, w, x, "sigmoid")
    assert np.allclose(y, s, rtol=4e-16, atol=0)
    y, _, _ = oracle.reference("q4b32", N, K, w, x, "silu_mul", m=m)
    assert np.allclose(y, xd * s * m, rtol=1e-15, atol=0)


# ----------------------------------------------------------------- metric

def test_metric_zero_for_exact_and_scaled_for_perturbation():
    rng = np.random.default_rng(41)
    acc = rng.normal(size=100)
    absacc = np.abs(acc) + rng.uniform(1, 2, size=100)
    res = compare(acc, acc, acc, absacc, "none")
    assert res["max_err"] == 0.0
    g = acc + 1e-5 * absacc
    assert compare(g, acc, acc, absacc, "none")["max_err"] == pytest.approx(1e-5, rel=1e-9)
    # near-zero outputs are judged against D, not |y|
    y0 = np.zeros(4)
    res = compare(np.full(4, 3e-6), y0, y0, np.full(4, 1.0), "none")
    assert res["max_err"] == pytest.approx(3e-6) and res["max_plain_rel"] == np.inf


def _fd(f, a, h):
    """Richardson-extrapolated central difference of f at a (error O(h^4))."""
    d1 = (f(a + h) - f(a - h)) / (2.0 * h)
    d2 = (f(a + h / 2) - f(a - h / 2)) / h
    return (4.0 * d2 - d1) / 3.0


# silu'(a) = 0 where 1 + a + e^a = 0, i.e. a = -1 - W(1/e) (W: Lambert's function)
SILU_STATIONARY = -1.2784645427610738
FD_POINTS = np.concatenate([np.linspace(-30.0, 30.0, 121), [SILU_STATIONARY, 1e-3, -1e-3, 0.0]])


def _d_sigmoid(a):
    """Numerical derivative of the oracle's own sigmoid.  Right of 0 the
    oracle's value is 1 - tiny and a difference there cancels, so the
    derivative is taken at -a, where the values are small and carry full
    precision (the logistic's derivative is even)."""
    b = -abs(a)
    return _fd(oracle.sigmoid, b, 1e-3 * max(1.0, abs(b)))


def _d_silu(a):
    return _fd(oracle.silu, a, 1e-3 * max(1.0, abs(a)))


def test_metric_error_scales_match_finite_differences():
    """D (oracle/compare.py, error_scale) is |dy/da| A, the first-order effect
    of the dot product's rounding on the output: checked for every epilogue
    against numerical derivatives of the oracle's own C sigmoid and silu (not
    a restatement of the formulas), at a in [-30, 30], silu's stationary point
    and around 0, to 1e-6 relative."""
    A = 3.7
    m, r = np.float32(-0.625), np.float32(1.5)
    for a in FD_POINTS:
        aa, AA = np.array([a]), np.array([A])
        cases = {
            "none": A * abs(_fd(lambda t: t, a, 1e-3)),
            "sigmoid": A * abs(_d_sigmoid(a)),
            "silu": A * abs(_d_silu(a)),
            "silu_mul": A * abs(_fd(lambda t: oracle.silu(t) * float(m), a, 1e-3 * max(1.0, abs(a)))),
            "mul": A * abs(_fd(lambda t: t * float(m), a, 1e-3)),
        }
        for act, want in cases.items():
            got = error_scale(act, aa, AA, m=np.array([m]), r=None)[0]
            if act in ("silu", "silu_mul") and abs(a - SILU_STATIONARY) < 1e-9:
                # silu' = 0 there: both sides vanish (the difference quotient
                # down to its own truncation error)
                assert got < 1e-12 * A and want < 1e-12 * A, (act, a, got, want)
                continue
            assert got == pytest.approx(want, rel=1e-6, abs=1e-300), (act, a, got, want)
        # add: the derivative part A plus |r|, the magnitude the final float32
        # addition rounds against
        got = error_scale("add", aa, AA, r=np.array([r]))[0]
        assert got - abs(float(r)) == pytest.approx(A * abs(_fd(lambda t: t + float(r), a, 1e-3)), rel=1e-6)


def test_metric_error_scale_catches_planted_derivative_slips():
    """A sign slip in silu' (s (1 - a (1 - s))) or a sigmoid' written s (1 + s)
    differs from the numerical derivatives by far more than the 1e-6 the pin
    allows, away from a = 0 where they happen to agree."""
    for a in (-4.0, -1.0, 2.5, 7.0):
        s = 1.0 / (1.0 + np.exp(-a))
        assert abs(abs(s * (1.0 - a * (1.0 - s))) - abs(_d_silu(a))) > 1e-3 * abs(_d_silu(a))
        assert abs(s * (1.0 + s) - abs(_d_sigmoid(a))) > 1e-3 * abs(_d_sigmoid(a))


def test_glu_metric_scale_matches_finite_differences():
    """glu_error_scale is |dy/dg| A_g + |dy/du| A_u for y = f(g) u, checked
    against numerical partial derivatives of the oracle's own silu and
    sigmoid."""
    Ag, Au = 2.25, 0.8
    f = {"silu": oracle.silu, "sigmoid": oracle.sigmoid}
    for act in ("silu", "sigmoid"):
        for g in FD_POINTS:
            for u in (-3.0, 0.5, 11.0):
                if act == "sigmoid":
                    dg = abs(_d_sigmoid(g) * u)
                else:
                    dg = abs(_fd(lambda t: f[act](t) * u, g, 1e-3 * max(1.0, abs(g))))
                du = abs(_fd(lambda t: f[act](g) * t, u, 1e-3 * max(1.0, abs(u))))
                want = dg * Ag + du * Au
                got = glu_error_scale(act, np.array([g]), np.array([Ag]), np.array([u]), np.array([Au]))[0]
                assert got == pytest.approx(want, rel=1e-6), (act, g, u, got, want)


def _gpu_order_f32(w, x):
    """float32 evaluation of W x in the vector-ALU kernels' documented order:
    lane l sums its 16-byte chunks l, l + 64, ... (E values each) with one
    rounding per product added, then the 64 lane sums meet pairwise in a
    6-level tree.  A model of the order on the CPU, sharing nothing with the
    kernels; numpy float64 products of float32 values are exact, each sum is
    rounded to float32."""
    N, K = w.shape
    E = 8
    nch = -(-K // E)
    out = np.zeros(N, np.float32)
    for i in range(N):
        lanes = np.zeros(64, np.float32)
        for c in range(nch):
            l = c % 64
            a = np.float32(lanes[l])
            for e in range(c * E, min(K, c * E + E)):
                a = np.float32(np.float64(a) + np.float64(w[i, e]) * np.float64(x[e]))
            lanes[l] = a
        v = lanes
        while v.size > 1:
            v = (v[: v.size // 2].astype(np.float64) + v[v.size // 2:].astype(np.float64)).astype(np.float32)
        out[i] = v[0]
    return out


def test_health_gate_passes_a_correct_order_and_fails_a_dropped_weight():
    """The health ratio (oracle/compare.py): a float32 evaluation in the
    kernels' summation order sits inside HEALTH_C * depth * 2^-24, while a
    result with a single weight dropped -- which the per-format f16 tolerance
    of 2e-3 still accepts -- lands far outside it."""
    rng = np.random.default_rng(51)
    N, K = 24, 4096
    wv = synth.random_weights(rng, "f16", N, K)
    w16 = wv.data.view(np.float16).reshape(N, K).astype(np.float64)
    x = synth.draw_vec(rng, K)
    y, acc, absacc = oracle.reference("f16", N, K, wv.data, x, "none")
    depth = -(-K // (64 * 8)) * (8 + 2) + 6
    g = _gpu_order_f32(w16, x)
    res = compare(g, y, acc, absacc, "none")
    assert res["max_err"] <= health_bound(depth)
    assert res["max_err"] / (depth * 2.0 ** -24) < 1.0  # the health ratio: O(1)
    # drop a typical term of row 5 (its magnitude the row's median |w x|)
    t = np.abs(w16[5] * x)
    j = int(np.argsort(t)[K // 2])
    w_drop = w16.copy()
    w_drop[5, j] = 0.0
    bad = (w_drop @ x.astype(np.float64)).astype(np.float32)
    res_bad = compare(bad, y, acc, absacc, "none")
    assert res_bad["max_err"] <= TOLERANCE["f16"]  # the spec gate alone misses it
    assert res_bad["max_err"] > 3 * health_bound(depth)
    assert res_bad["argmax"] == 5


def test_float32_rounding_of_oracle_passes_metric():
    """The oracle's own result rounded to float32 sits far inside every tolerance."""
    for wl in (synth.f32_tiny_256(0),):
        for c in wl.calls:
            w = wl.weights[c.w]
            m = wl.vectors.get(c.m) if c.m else None
            r = wl.vectors.get(c.r) if c.r else None
            y, acc, absacc = oracle.reference(w.fmt, w.N, w.K, w.data, wl.vectors[c.x], c.act, m=m, r=r)
            res = compare(y.astype(np.float32), y, acc, absacc, c.act, m=m, r=r)
            assert res["max_err"] < TOLERANCE[w.fmt] * 1e-1


# ----------------------------------------------------------------- planted mistakes

def test_pins_catch_planted_mistakes(golden_dir):
    """Plant plausible mistakes in the oracle's outputs on the CPU and show that
    the pins above would reject them."""
    fx = json.load(open(os.path.join(golden_dir, "q4b32_blocks.json")))
    good = oracle.decode("q4b32", 2, 64, _image(fx))
    want0 = np.array([float(Fraction(s)) for s in fx["expected_row0"]])
    assert np.array_equal(good[0], want0)
    swapped = good[0].reshape(-1, 2)[:, ::-1].reshape(-1)          # nibble order swapped
    assert not np.array_equal(swapped, want0)
    no_offset = good[0] + 8.0                                       # dropped the -8
    assert not np.array_equal(no_offset, want0)
    # wrong sigmoid sign: 1/(1+exp(a)) fails the closed form sigma(ln 3) = 3/4
    assert abs(1.0 / (1.0 + math.exp(math.log(3.0))) - 0.75) > 0.1
    # transposed operand fails the non-square rank-1 pin (shape alone differs)
    rng = np.random.default_rng(43)
    W = rng.normal(size=(5, 12)).astype(np.float32)
    x = rng.normal(size=12).astype(np.float32)
    acc, _ = oracle.gemv("f32", 5, 12, W.view(np.uint8), x)
    with pytest.raises(ValueError):
        oracle.gemv("f32", 12, 5, W.T.copy().view(np.uint8), x)
    assert acc.shape == (5,)


def test_metric_subnormal_floor():
    """Outputs below the smallest normal float32 are judged in absolute terms
    against 2^-126 (float32 has only absolute precision there)."""
    y = np.array([1e-45, -3e-40])
    g = np.array([0.0, -2.9e-40])
    res = compare(g, y, np.array([1e-45, -3e-40]), np.array([1e-50, 1e-50]), "none")
    assert res["max_err"] == pytest.approx(1e-41 / 2.0 ** -126, rel=1e-9)


# ----------------------------------------------------------------- gated pair (GLU)

def test_glu_closed_forms():
    """Zero gate: silu(0) = 0 gives 0 and sigmoid(0) = 1/2 gives u/2; zero up
    gives 0; identity gate with scipy's logistic."""
    rng = np.random.default_rng(51)
    N = K = 64
    x = synth.draw_vec(rng, K)
    wu = synth.random_weights(rng, "f16", N, K)
    zero = np.zeros(N * K, dtype=np.float16).view(np.uint8)
    u, _ = oracle.gemv("f16", N, K, wu.data, x)
    y, *_ = oracle.glu_reference("f16", N, K, zero, wu.data, x, "silu")
    assert np.all(y == 0.0)
    y, *_ = oracle.glu_reference("f16", N, K, zero, wu.data, x, "sigmoid")
    assert np.array_equal(y, 0.5 * u)
    y, *_ = oracle.glu_reference("f16", N, K, wu.data, zero, x, "silu")
    assert np.all(y == 0.0)
    eye = np.eye(N, K, dtype=np.float16).view(np.uint8).reshape(-1)
    y, *_ = oracle.glu_reference("f16", N, K, eye, wu.data, x, "silu")
    xd = x.astype(np.float64)
    assert np.allclose(y, xd * scipy.special.expit(xd) * u, rtol=1e-15, atol=0)
    y, *_ = oracle.glu_reference("f16", N, K, eye, wu.data, x, "sigmoid")
    assert np.allclose(y, scipy.special.expit(xd) * u, rtol=1e-15, atol=0)
    with pytest.raises(ValueError):
        oracle.glu_epilogue("add", u, u)


def test_glu_ncols_closed_forms_and_column_order():
    """Identity gate and up over several columns: column b is act(x_b) * x_b
    (scipy's logistic); zero up gives 0 everywhere; reversing the columns of X
    reverses the columns of the result; one column is the one-column pair."""
    rng = np.random.default_rng(52)
    N = K = 64
    B = 5
    X = np.stack([synth.draw_vec(rng, K) for _ in range(B)])
    eye = np.eye(N, K, dtype=np.float16).view(np.uint8).reshape(-1)
    zero = np.zeros(N * K, dtype=np.float16).view(np.uint8)
    Xd = X.astype(np.float64)
    Y, G, _, U, _ = oracle.glu_ncols_reference("f16", N, K, eye, eye, X, "silu")
    assert np.allclose(Y, Xd * scipy.special.expit(Xd) * Xd, rtol=1e-15, atol=0)
    assert np.array_equal(G, Xd) and np.array_equal(U, Xd)
    Y, *_ = oracle.glu_ncols_reference("f16", N, K, eye, eye, X, "sigmoid")
    assert np.allclose(Y, scipy.special.expit(Xd) * Xd, rtol=1e-15, atol=0)
    Y, *_ = oracle.glu_ncols_reference("f16", N, K, eye, zero, X, "silu")
    assert np.all(Y == 0.0)
    wg = synth.random_weights(rng, "q4b32", N, K)
    wu = synth.random_weights(rng, "q4b32", N, K)
    Y, *_ = oracle.glu_ncols_reference("q4b32", N, K, wg.data, wu.data, X, "silu")
    Yr, *_ = oracle.glu_ncols_reference("q4b32", N, K, wg.data, wu.data, X[::-1], "silu")
    assert np.array_equal(Yr, Y[::-1])
    y1, *_ = oracle.glu_reference("q4b32", N, K, wg.data, wu.data, X[2], "silu")
    Y1, *_ = oracle.glu_ncols_reference("q4b32", N, K, wg.data, wu.data, X[2:3], "silu")
    assert np.array_equal(Y1[0], y1)
    Ys, *_ = oracle.glu_ncols_reference("q4b32", N, K, wg.data, wu.data, X, "silu", rows=(7, 30))
    assert np.array_equal(Ys, Y[:, 7:30])


# ----------------------------------------------------------------- several columns (ncols)

@pytest.mark.parametrize("fmt,N,K,B", [("f32", 3, 7, 3), ("f16", 4, 13, 2), ("q4b32", 3, 64, 4),
                                       ("q8b32", 2, 32, 8)])
def test_ncols_brute_force_exact(fmt, N, K, B):
    """Each destination column against exact rational arithmetic over the
    whole [ncols, K] input, and the residual add in the b-major layout."""
    rng = np.random.default_rng(N * 100 + K + B)
    w = synth.random_weights(rng, fmt, N, K)
    X = rng.normal(size=(B, K)).astype(np.float32)
    Rr = rng.normal(size=(B, N)).astype(np.float32)
    Y, acc, absacc = oracle.ncols_reference(fmt, N, K, w.data, X, "add", R=Rr)
    assert Y.shape == acc.shape == absacc.shape == (B, N)
    ex = _exact_values(w)
    for b in range(B):
        xf = [Fraction(float(v)) for v in X[b]]
        for i in range(N):
            exact = sum(ex[i][j] * xf[j] for j in range(K))
            A = sum(abs(ex[i][j] * xf[j]) for j in range(K))
            bound = gamma(max(K - 1, 0)) * float(A)
            assert abs(float(Fraction(acc[b, i]) - exact)) <= bound * (1 + 1e-12) + 1e-300
            assert abs(float(Fraction(absacc[b, i]) - A)) <= bound * (1 + 1e-12) + 1e-300
            y_exact = exact + Fraction(float(Rr[b, i]))
            assert abs(float(Fraction(Y[b, i]) - y_exact)) <= (bound + U * abs(float(y_exact))) * (1 + 1e-9) + 1e-300


def _one_hot_columns(B, K, rng):
    cols = rng.choice(K, size=B, replace=False)
    X = np.zeros((B, K), dtype=np.float32)
    X[np.arange(B), cols] = 1.0
    return X, cols


def test_ncols_one_hot_selects_weight_columns():
    """x_b = e_{j_b}: column b of the output is column j_b of W exactly, and
    the multiply tail takes its operand from row b of M (b-major)."""
    rng = np.random.default_rng(61)
    N, K, B = 40, 96, 5
    w = synth.random_weights(rng, "q4b32", N, K)
    X, cols = _one_hot_columns(B, K, rng)
    M = rng.normal(size=(B, N)).astype(np.float32)
    dense = (w.codes.astype(np.float64) - 8.0) * np.repeat(w.scales.astype(np.float64), 32, axis=1)
    Y, acc, _ = oracle.ncols_reference("q4b32", N, K, w.data, X, "mul", M=M)
    for b in range(B):
        assert np.array_equal(acc[b], dense[:, cols[b]])
        assert np.array_equal(Y[b], dense[:, cols[b]] * M[b].astype(np.float64))


def test_ncols_single_column_rows_and_zero_x():
    """One column reproduces the one-column result on any row slice; x = 0
    gives epilogue(0) per column (ADD returns the residual row of its column)."""
    rng = np.random.default_rng(62)
    N, K, B = 33, 64, 3
    w = synth.random_weights(rng, "bf16", N, K)
    X = np.zeros((B, K), dtype=np.float32)
    Rr = rng.normal(size=(B, N)).astype(np.float32)
    Y, acc, _ = oracle.ncols_reference("bf16", N, K, w.data, X, "add", R=Rr)
    assert np.all(acc == 0.0) and np.array_equal(Y, Rr.astype(np.float64))
    Y, *_ = oracle.ncols_reference("bf16", N, K, w.data, X, "sigmoid", rows=(5, 20))
    assert Y.shape == (B, 15) and np.all(Y == 0.5)


def test_ncols_pins_catch_transposed_operand():
    """A plausible layout mistake -- reading the [ncols, N] operand as
    [N, ncols] -- fails the one-hot pin."""
    rng = np.random.default_rng(63)
    N, K, B = 24, 32, 3
    w = synth.random_weights(rng, "f32", N, K)
    X, cols = _one_hot_columns(B, K, rng)
    M = rng.normal(size=(B, N)).astype(np.float32)
    dense = w.data.view(np.float32).reshape(N, K).astype(np.float64)
    wrong = M.reshape(N, B).T.copy()  # the mistaken reading
    Y, *_ = oracle.ncols_reference("f32", N, K, w.data, X, "mul", M=wrong)
    assert any(not np.array_equal(Y[b], dense[:, cols[b]] * M[b].astype(np.float64)) for b in range(B))


# ----------------------------------------------------------------- signed Hadamard transform

def test_fwht_small_closed_forms():
    """n = 1 is the sign multiply; n = 2 is (a + b, a - b) / sqrt 2; the 4-point
    case worked by hand (signs broadcast with period 2)."""
    x = np.array([3.0, -5.0, 7.0], np.float32)
    y, d = oracle.fwht_signed(x, np.array([-1.0], np.float32), 1)
    assert np.array_equal(y, -x.astype(np.float64)) and np.array_equal(d, np.abs(x).astype(np.float64))
    y, _ = oracle.fwht_signed(np.array([2.0, 1.0], np.float32), np.array([1.0, 1.0], np.float32), 2)
    assert np.allclose(y, [3 / math.sqrt(2), 1 / math.sqrt(2)], rtol=1e-15, atol=0)
    y, d = oracle.fwht_signed(np.array([1, 2, 3, 4], np.float32), np.array([1, -1], np.float32), 4)
    # (1, -2, 3, -4) against the rows of H_4, over 2
    assert np.array_equal(y, [-1.0, 5.0, 0.0, -2.0]) and np.array_equal(d, [5.0] * 4)


@pytest.mark.parametrize("n", [2, 8, 64, 1024])
def test_fwht_against_scipy_hadamard(n):
    """Sylvester's matrix from scipy (a library routine) times x * s, over
    sqrt(n), block by block."""
    import scipy.linalg
    rng = np.random.default_rng(n)
    K = 3 * n
    x = rng.normal(size=K).astype(np.float32)
    s = rng.choice([-1.0, 1.0], size=n).astype(np.float32)
    y, d = oracle.fwht_signed(x, s, n)
    H = scipy.linalg.hadamard(n).astype(np.float64) / math.sqrt(n)
    v = (x.astype(np.float64) * np.tile(s, 3)).reshape(3, n)
    want = (v @ H.T).reshape(-1)
    assert np.all(np.abs(y - want) <= 4 * n * U * d)


def test_fwht_unit_vectors_give_sylvester_columns():
    """x = e_j gives column j of H_n / sqrt(n): (-1)^popcount(i & j) / sqrt(n).
    This fixes the natural (Sylvester) order against a sequency (Walsh) order."""
    n = 16
    for j in (0, 1, 5, 10, 15):
        x = np.zeros(n, np.float32)
        x[j] = 1.0
        y, _ = oracle.fwht_signed(x, np.ones(1, np.float32), n)
        want = np.array([(-1.0) ** bin(i & j).count("1") for i in range(n)]) / 4.0
        assert np.array_equal(y, want), j


def test_fwht_parseval_and_involution():
    """Orthonormal: the sum of squares is kept, and the unsigned transform
    applied twice gives back x * s."""
    rng = np.random.default_rng(71)
    n, K = 256, 1024
    x = rng.normal(size=K).astype(np.float32)
    s = rng.choice([-1.0, 1.0], size=K).astype(np.float32)
    y, d = oracle.fwht_signed(x, s, n)
    xs = x.astype(np.float64) * s
    assert abs(np.sum(y * y) - np.sum(xs * xs)) <= 1e-12 * np.sum(xs * xs)
    y2, _ = oracle.fwht_signed(y.astype(np.float32), np.ones(1, np.float32), n)
    # y rounded to float32 before the second pass: error of order 2^-24 |y|
    assert np.max(np.abs(y2 - xs)) <= 1e-6 * np.max(np.abs(xs))


def test_fwht_sign_broadcast_period():
    """The sign of element k is s[k mod len(s)]: a period-3 sign vector over
    K = 12 (blocks of 4) against the same signs written out at full length."""
    rng = np.random.default_rng(72)
    x = rng.normal(size=12).astype(np.float32)
    s3 = np.array([1.0, -1.0, -1.0], np.float32)
    y, _ = oracle.fwht_signed(x, s3, 4)
    y_full, _ = oracle.fwht_signed(x, np.tile(s3, 4), 4)
    assert np.array_equal(y, y_full)
    # a plausible mistake -- indexing the signs within the block, k mod n --
    # gives a different result here
    wrong, _ = oracle.fwht_signed(x, np.tile(np.tile(s3, 2)[:4], 3), 4)
    assert not np.array_equal(y, wrong)
    with pytest.raises(ValueError):
        oracle.fwht_signed(x, np.ones(5, np.float32), 4)   # 5 does not divide 12
    with pytest.raises(ValueError):
        oracle.fwht_signed(x, np.ones(1, np.float32), 3)   # not a power of two


def test_fwht_pins_catch_dropped_scale():
    """Without the 1/sqrt(n) scale the transform is not orthonormal: Parseval
    fails by a factor n."""
    rng = np.random.default_rng(73)
    n = 64
    x = rng.normal(size=n).astype(np.float32)
    y, _ = oracle.fwht_signed(x, np.ones(1, np.float32), n)
    unscaled = y * math.sqrt(n)
    assert abs(np.sum(unscaled ** 2) / np.sum(x.astype(np.float64) ** 2) - n) < 1e-9


def test_fwht_gemv_reference_composition():
    """The transform feeds the product: with W = the transform's own matrix
    (f32, n = K = 32, signs +1), W x' = H (H x) / n = x, up to the float32
    rounding of x'; the error scale covers it."""
    import scipy.linalg
    n = K = 32
    rng = np.random.default_rng(74)
    x = rng.normal(size=K).astype(np.float32)
    H = (scipy.linalg.hadamard(n) / math.sqrt(n)).astype(np.float32)
    y, acc, absacc = oracle.fwht_gemv_reference("f32", n, K, H.view(np.uint8).reshape(-1), x,
                                                np.ones(1, np.float32), n, "none")
    assert np.all(np.abs(y - x) <= 1e-6 * absacc)
    assert np.all(absacc >= np.abs(acc))
