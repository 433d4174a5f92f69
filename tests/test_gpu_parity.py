"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by
element on the same seeded inputs, with the per-format tolerances of the
guarded error metric (1e-5 f32, 2e-3 f16/bf16, 1e-4 block formats)."""
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from decode_gemv_elementwise_amd import binding, synth
from gpu_util import assert_healthy, check_ncols, check_parity, dev, host, log, run_fused
from oracle.compare import TOLERANCE, compare

pytestmark = pytest.mark.gpu

ALL_ACTS = list(synth.ACTS)


def _operands(rng, act, N):
    m = synth.draw_vec(rng, N) if act in ("silu_mul", "mul") else None
    r = synth.draw_vec(rng, N) if act == "add" else None
    return m, r


# ------------------------------------------------------------------ workloads at full size

def _resolve(wl, name, outputs):
    if name is None:
        return None
    if name.startswith("@"):
        return outputs[name[1:]]
    return wl.vectors[name]


@pytest.mark.parametrize("wname", list(synth.WORKLOADS))
def test_workload_calls_full_size(wname):
    """Every call of every workload at its full size; all rows compared.  A
    chained input (the multiplier of the up projection, the input of the down
    projection) is the oracle's own f32-rounded output of the earlier call, fed
    to both sides."""
    wl = synth.WORKLOADS[wname](0)
    outputs = {}
    for c in wl.calls:
        w = wl.weights[c.w]
        x = _resolve(wl, c.x, outputs)
        m = _resolve(wl, c.m, outputs)
        r = _resolve(wl, c.r, outputs)
        if c.w2 and c.ncols > 1:
            from test_gpu_glu_ncols import _check as check_glu_ncols
            X = np.reshape(x, (c.ncols, w.K))
            check_glu_ncols(w, wl.weights[c.w2], X, c.act, f"{wname}/{c.name}")
            y = oracle.glu_ncols_reference(w.fmt, w.N, w.K, w.data, wl.weights[c.w2].data, X, c.act)[0].reshape(-1)
        elif c.w2:
            check_glu(w, wl.weights[c.w2], x, c.act, f"{wname}/{c.name}")
            y = oracle.glu_reference(w.fmt, w.N, w.K, w.data, wl.weights[c.w2].data, x, c.act)[0]
        elif c.fwht:
            from test_gpu_fwht import check_fused_fwht
            sg = wl.vectors[c.fwht[0]]
            check_fused_fwht(w, x, sg, c.fwht[1], c.act, m=m, r=r, tag=f"{wname}/{c.name}",
                             out_shape=c.out_shape, inplace=c.inplace)
            y = oracle.fwht_gemv_reference(w.fmt, w.N, w.K, w.data, x, sg, c.fwht[1], c.act, m=m, r=r)[0]
        elif c.ncols > 1:
            X = np.reshape(x, (c.ncols, w.K))
            M = None if m is None else np.reshape(m, (c.ncols, w.N))
            R = None if r is None else np.reshape(r, (c.ncols, w.N))
            shape = c.out_shape or (c.ncols, w.N)
            check_ncols(w, X, c.act, M, R, out_shape=shape, inplace=c.inplace, tag=f"{wname}/{c.name}")
            y = oracle.ncols_reference(w.fmt, w.N, w.K, w.data, X, c.act, M=M, R=R)[0].reshape(-1)
        else:
            g, y, res = check_parity(w, x, c.act, m=m, r=r, out_shape=c.out_shape, inplace=c.inplace,
                                     tag=f"{wname}/{c.name}")
            log(f"  {c.name}: max_err={res['max_err']:.2e} plain_rel={res['max_plain_rel']:.2e}")
        outputs[c.name] = y.astype(np.float32)


# ------------------------------------------------------------------ every format x epilogue

@pytest.mark.parametrize("fmt", synth.FORMATS)
@pytest.mark.parametrize("act", ALL_ACTS)
def test_format_epilogue_matrix(fmt, act):
    rng = np.random.default_rng(zlib.crc32(f"{fmt}/{act}".encode()))
    N, K = 300, 512
    w = synth.random_weights(rng, fmt, N, K)
    x = synth.draw_vec(rng, K)
    m, r = _operands(rng, act, N)
    check_parity(w, x, act, m=m, r=r, tag=f"matrix {fmt}/{act}")


# ------------------------------------------------------------------ odd, ragged and extreme shapes

# The largest K whose staged x fits the 160 KiB of LDS a workgroup may take,
# and the next one (the generic kernel): f32 40960 / 40964, f16 and bf16
# 27304 / 27312 (12 floats of LDS per 8 values), 8-bit 32768 / 32800, 4-bit
# 36384 / 36416.
FLOAT_SHAPES = [(1, 1), (1, 7), (3, 64), (5, 4), (33, 257), (64, 1000), (17, 4097), (4097, 33),
                (1000, 256), (1003, 4096), (300, 8192), (67, 14336), (2, 27304), (2, 27312), (2, 40960),
                (2, 40964), (65539, 8)]
BLOCK_SHAPES = [(1, 32), (7, 64), (33, 96), (1000, 4096), (3, 32000), (2, 32768), (2, 32800), (2, 36384),
                (2, 36416), (1, 65536), (4099, 32)]


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("N,K", FLOAT_SHAPES)
def test_float_shapes(fmt, N, K):
    rng = np.random.default_rng(N * 7919 + K)
    w = synth.random_weights(rng, fmt, N, K)
    x = synth.draw_vec(rng, K)
    r = synth.draw_vec(rng, N)
    check_parity(w, x, "add", r=r, tag=f"shape {fmt} {N}x{K}")


@pytest.mark.parametrize("fmt", ["q8b32", "q4b32"])
@pytest.mark.parametrize("N,K", BLOCK_SHAPES)
def test_block_shapes(fmt, N, K):
    rng = np.random.default_rng(N * 7919 + K + 1)
    w = synth.random_weights(rng, fmt, N, K)
    x = synth.draw_vec(rng, K)
    check_parity(w, x, "silu", tag=f"shape {fmt} {N}x{K}")


# ------------------------------------------------------------------ exact cases

def test_integer_exact_q8():
    """Scale 1 and small integer x: every partial sum is an integer below 2^24,
    so any summation order gives the same value: GPU == oracle bit for bit."""
    log("integer exact q8")
    rng = np.random.default_rng(3)
    N, K = 1024, 6144
    codes = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    w = synth.Weights("q8b32", N, K, synth.pack_q8b32(codes, np.ones((N, K // 32), np.float16)))
    x = rng.integers(-3, 4, size=K).astype(np.float32)
    g, _ = run_fused(w, x, "none")
    acc, _ = oracle.gemv("q8b32", N, K, w.data, x)
    assert np.array_equal(g.astype(np.float64), acc)


def test_integer_exact_q4_and_f16():
    log("integer exact q4 / f16")
    rng = np.random.default_rng(4)
    N, K = 512, 4096
    codes = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    w = synth.Weights("q4b32", N, K, synth.pack_q4b32(codes, np.ones((N, K // 32), np.float16)))
    x = rng.integers(-4, 5, size=K).astype(np.float32)
    g, _ = run_fused(w, x, "none")
    acc, _ = oracle.gemv("q4b32", N, K, w.data, x)
    assert np.array_equal(g.astype(np.float64), acc)
    Wf = rng.integers(-8, 9, size=(N, K)).astype(np.float16)
    wf = synth.Weights("f16", N, K, Wf.view(np.uint8).reshape(-1))
    g, _ = run_fused(wf, x, "none")
    acc, _ = oracle.gemv("f16", N, K, wf.data, x)
    assert np.array_equal(g.astype(np.float64), acc)


def _integer_weights(rng, fmt, N, K):
    """Small integers, exact in every float format."""
    W = rng.integers(-8, 9, size=(N, K))
    if fmt == "f32":
        data = W.astype(np.float32).view(np.uint8).reshape(-1)
    elif fmt == "f16":
        data = W.astype(np.float16).view(np.uint8).reshape(-1)
    else:  # bf16: the upper half of the float32 pattern, exact for |w| <= 256
        data = (W.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16).view(np.uint8).reshape(-1)
    return synth.Weights(fmt, N, K, data)


@pytest.mark.parametrize("fmt,N,K", [("bf16", 512, 4096), ("f32", 512, 4096), ("bf16", 64, 14336),
                                     ("f16", 96, 4097), ("f32", 7, 40964), ("bf16", 33, 1000),
                                     ("f32", 1000, 257)])
def test_integer_exact_float_formats(fmt, N, K):
    """Integer weights and x in {-3..3}: every partial sum, in any order, is
    an integer below 2^24, so the float32 result equals the oracle's double
    sum bit for bit -- on aligned rows (the chunked kernel) and on ragged K
    (4097: f16 rows that are not whole 16-byte chunks; 40964: f32 x too long
    to stage, both on the element-wise kernel), for every epilogue that keeps
    integers (none, mul by an integer, add an integer)."""
    log(f"integer exact {fmt} {N}x{K}")
    rng = np.random.default_rng(N + K)
    w = _integer_weights(rng, fmt, N, K)
    x = rng.integers(-3, 4, size=K).astype(np.float32)
    acc, _ = oracle.gemv(fmt, N, K, w.data, x)
    assert np.all(np.abs(acc) < 2 ** 24)
    g, _ = run_fused(w, x, "none")
    assert np.array_equal(g.astype(np.float64), acc)
    mi = rng.integers(-5, 6, size=N).astype(np.float32)
    g, _ = run_fused(w, x, "mul", m=mi)
    assert np.array_equal(g.astype(np.float64), acc * mi)
    g, _ = run_fused(w, x, "add", r=mi)
    assert np.array_equal(g.astype(np.float64), acc + mi)


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_zero_weights(fmt):
    log(f"zero W {fmt}")
    N, K = 130, 256
    nb = synth.weight_nbytes(fmt, N, K)
    data = np.zeros(nb, dtype=np.uint8)
    if fmt == "q4b32":  # code 8 is value 0
        data[: N * K // 2] = 0x88
    w = synth.Weights(fmt, N, K, data)
    rng = np.random.default_rng(1)
    x = synth.draw_vec(rng, K)
    m = synth.draw_vec(rng, N)
    r = synth.draw_vec(rng, N)
    want = {"none": 0.0, "sigmoid": 0.5, "silu": 0.0, "silu_mul": 0.0, "mul": 0.0}
    for act, v in want.items():
        g, _ = run_fused(w, x, act, m=m if act in ("silu_mul", "mul") else None)
        assert np.all(g == v), (fmt, act)
    g, _ = run_fused(w, x, "add", r=r)
    assert np.array_equal(g, r)


def test_identity_weights():
    """4-bit identity (code 9 on the diagonal, 8 elsewhere, scale 1): the
    accumulator is x exactly, so NONE returns x bit for bit."""
    log("identity q4")
    N = K = 4096
    codes = np.full((N, K), 8, dtype=np.uint8)
    np.fill_diagonal(codes, 9)
    w = synth.Weights("q4b32", N, K, synth.pack_q4b32(codes, np.ones((N, K // 32), np.float16)))
    x = synth.draw_vec(np.random.default_rng(2), K)
    g, _ = run_fused(w, x, "none")
    assert np.array_equal(g, x)
    check_parity(w, x, "sigmoid", tag="identity sigmoid")


# ------------------------------------------------------------------ fused == unfused, determinism

def _fused_and_unfused(w, x, act, m, r):
    Wd, xd = dev(w.data), dev(x)
    md = dev(m) if m is not None else None
    rd = dev(r) if r is not None else None
    fused = torch.empty(w.N, dtype=torch.float32, device="cuda")
    binding.gemv_fused(Wd, w.fmt, w.N, w.K, xd, act, mul_operand=md, add_operand=rd, dst=fused)
    tmp = torch.empty(w.N, dtype=torch.float32, device="cuda")
    unfused = torch.empty(w.N, dtype=torch.float32, device="cuda")
    binding.gemv_fused(Wd, w.fmt, w.N, w.K, xd, "none", dst=tmp)
    binding.gemv_epilogue(act, w.N, tmp, mul_operand=md, add_operand=rd, dst=unfused)
    torch.cuda.synchronize()
    return host(fused), host(unfused)


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_fused_equals_unfused_bitwise(fmt):
    """The fused epilogue and the separate element-wise pass give identical
    bits for every epilogue (ADD and MUL must; here SIGMOID/SILU/SILU_MUL do
    too, since both paths run the same device function on the same value)."""
    rng = np.random.default_rng(11)
    N, K = 4099, 1024
    w = synth.random_weights(rng, fmt, N, K)
    x = synth.draw_vec(rng, K)
    for act in ALL_ACTS:
        log(f"fused==unfused {fmt} {act}")
        m, r = _operands(rng, act, N)
        f, u = _fused_and_unfused(w, x, act, m, r)
        assert np.array_equal(f.view(np.uint32), u.view(np.uint32)), (fmt, act)


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_deterministic(fmt):
    log(f"determinism {fmt}")
    rng = np.random.default_rng(12)
    N, K = 2048, 4096
    w = synth.random_weights(rng, fmt, N, K)
    x = synth.draw_vec(rng, K)
    a, _ = run_fused(w, x, "silu")
    b, _ = run_fused(w, x, "silu")
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ------------------------------------------------------------------ aliasing and views

def test_inplace_add_matches_out_of_place():
    log("in-place add")
    rng = np.random.default_rng(13)
    w = synth.random_weights(rng, "f16", 4096, 4096)
    x = synth.draw_vec(rng, 4096)
    r = synth.draw_vec(rng, 4096)
    g_in, _ = run_fused(w, x, "add", r=r, inplace=True)
    g_out, _ = run_fused(w, x, "add", r=r)
    assert np.array_equal(g_in, g_out)


def test_inplace_mul_and_view_add():
    log("in-place mul, [32,128] view add in place")
    rng = np.random.default_rng(14)
    w = synth.random_weights(rng, "q8b32", 4096, 6144)
    x = synth.draw_vec(rng, 6144)
    m = synth.draw_vec(rng, 4096)
    check_parity(w, x, "mul", m=m, inplace=True, tag="q8 mul in place")
    r = synth.draw_vec(rng, 4096).reshape(32, 128)
    check_parity(w, x, "add", r=r, out_shape=(32, 128), inplace=True, tag="q8 view add in place")


def test_rejected_call_writes_nothing():
    log("rejected calls")
    rng = np.random.default_rng(15)
    w = synth.random_weights(rng, "f32", 64, 64)
    Wd, xd = dev(w.data), dev(synth.draw_vec(rng, 64))
    dst = torch.full((64,), 7.0, dtype=torch.float32, device="cuda")
    r = torch.ones(64, dtype=torch.float32, device="cuda")
    with pytest.raises(binding.GemvError) as e:
        binding.gemv_fused(Wd, "f32", 64, 64, xd, "add", dst=dst)  # missing residual
    assert e.value.status == binding.STATUS_CODE["GEMV_E_OPERAND"]
    with pytest.raises(binding.GemvError) as e:
        binding.gemv_fused(Wd, "f32", 64, 64, xd, "add", add_operand=r[1:], dst=dst[:63])  # N mismatch
    assert e.value.status == binding.STATUS_CODE["GEMV_E_DIM"]
    with pytest.raises(binding.GemvError) as e:
        binding.gemv_fused(Wd, "f32", 64, 64, xd, 9, dst=dst)
    assert e.value.status == binding.STATUS_CODE["GEMV_E_ACT"]
    alias = torch.zeros(80, dtype=torch.float32, device="cuda")
    with pytest.raises(binding.GemvError) as e:  # dst shifted by one element against the residual
        binding.gemv_fused(Wd, "f32", 64, 64, xd, "add", add_operand=alias[:64], dst=alias[1:65])
    assert e.value.status == binding.STATUS_CODE["GEMV_E_ALIAS"]
    torch.cuda.synchronize()
    assert torch.all(dst == 7.0)
    assert torch.all(alias == 0.0)


def _separate_ops(w, Wd, xd, act, operand, dst):
    """What a caller does when a guard refuses the fused call: the separate
    ops ("vulkan: fuse the sign multiply into the Hadamard FWHT", Additional
    information; "ggml-cpu: fuse element-wise epilogues ...", Guards).  The
    product goes to scratch the caller owns, the operand to a contiguous
    buffer of dst's shape, then the element-wise pass writes dst."""
    tmp = torch.empty(w.N, dtype=torch.float32, device="cuda")
    binding.gemv_fused(Wd, w.fmt, w.N, w.K, xd, "none", dst=tmp)
    op = operand.expand(dst.shape).contiguous().clone()
    kw = {"add_operand": op} if act == "add" else {"mul_operand": op}
    binding.gemv_epilogue(act, w.N, tmp, dst=dst, **kw)
    torch.cuda.synchronize()


def test_guard_failure_falls_back_to_separate_ops():
    """A call the guards refuse writes nothing; the caller's separate ops then
    give the oracle's result, so only the speed changes, not the values."""
    rng = np.random.default_rng(16)
    cases = [
        # dst one element past the residual in one buffer: a shifted overlap
        ("f16", 4096, 4096, "add", "alias", binding.STATUS_CODE["GEMV_E_ALIAS"]),
        # every other element of a larger buffer: not contiguous
        ("q8b32", 4096, 6144, "mul", "strided", binding.STATUS_CODE["GEMV_E_LAYOUT"]),
        # one multiplier broadcast over every row: stride 0
        ("bf16", 1024, 4096, "silu_mul", "broadcast", binding.STATUS_CODE["GEMV_E_LAYOUT"]),
    ]
    for fmt, N, K, act, kind, status in cases:
        log(f"guard fallback {fmt} {N}x{K} {act} {kind}")
        w = synth.random_weights(rng, fmt, N, K)
        x = synth.draw_vec(rng, K)
        Wd, xd = dev(w.data), dev(x)
        if kind == "alias":
            buf = dev(np.concatenate([synth.draw_vec(rng, N), np.zeros(1, np.float32)]))
            operand, dst = buf[:N], buf[1:]
            values = host(operand).copy()
        elif kind == "strided":
            big = dev(synth.draw_vec(rng, 2 * N))
            operand = big[::2]
            dst = torch.full((N,), 7.0, dtype=torch.float32, device="cuda")
            values = host(operand).copy()
        else:
            operand = dev(synth.draw_vec(rng, 1)).expand(N)
            dst = torch.full((N,), 7.0, dtype=torch.float32, device="cuda")
            values = np.full(N, host(operand)[0], np.float32)
        before = host(dst).copy()
        kw = {"add_operand": operand} if act == "add" else {"mul_operand": operand}
        with pytest.raises(binding.GemvError) as e:
            binding.gemv_fused(Wd, fmt, N, K, xd, act, dst=dst, **kw)
        assert e.value.status == status, (kind, e.value.status)
        torch.cuda.synchronize()
        assert np.array_equal(host(dst), before), kind
        _separate_ops(w, Wd, xd, act, operand, dst)
        g = host(dst).reshape(-1)
        m = values if act != "add" else None
        r = values if act == "add" else None
        y, acc, absacc = oracle.reference(fmt, N, K, w.data, x, act, m=m, r=r)
        res = compare(g, y, acc, absacc, act, m=m, r=r)
        assert res["max_err"] <= TOLERANCE[fmt], (kind, res)


# ------------------------------------------------------------------ the 4-bit layer chain

def test_layer_chain_fused_vs_unfused_and_gate_up_pairing():
    """The six-GEMV 4-bit layer runs fused (6 launches) and unfused (6 GEMVs +
    5 element-wise passes = 11 launches) with identical final bits; and
    up * silu(gate) computed as MUL-after-SILU equals SILU_MUL-after-NONE."""
    log("layer chain")
    wl = synth.q4b32_decode_layer(0)
    Wd = {k: dev(w.data) for k, w in wl.weights.items()}
    V = {k: dev(v) for k, v in wl.vectors.items()}
    ws = wl.weights

    def f32(n):
        return torch.empty(n, dtype=torch.float32, device="cuda")

    def chain(fused: bool):
        outs = {}
        for c in wl.calls:
            w = ws[c.w]
            x = outs[c.x[1:]] if c.x.startswith("@") else V[c.x]
            m = (outs[c.m[1:]] if c.m.startswith("@") else V[c.m]) if c.m else None
            r = V[c.r] if c.r else None
            out = f32(w.N)
            if fused or c.act == "none":
                binding.gemv_fused(Wd[c.w], "q4b32", w.N, w.K, x, c.act, mul_operand=m, add_operand=r, dst=out)
            else:
                tmp = f32(w.N)
                binding.gemv_fused(Wd[c.w], "q4b32", w.N, w.K, x, "none", dst=tmp)
                binding.gemv_epilogue(c.act, w.N, tmp, mul_operand=m, add_operand=r, dst=out)
            outs[c.name] = out
        torch.cuda.synchronize()
        return {k: host(v) for k, v in outs.items()}

    a, b = chain(True), chain(False)
    for k in a:
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k

    # pairing: SILU on gate then MUL on up  ==  NONE on up then SILU_MUL on gate with m = up
    g, u = ws["Wgate"], ws["Wup"]
    up_raw = f32(u.N)
    binding.gemv_fused(Wd["Wup"], "q4b32", u.N, u.K, V["x_ffn"], "none", dst=up_raw)
    paired = f32(g.N)
    binding.gemv_fused(Wd["Wgate"], "q4b32", g.N, g.K, V["x_ffn"], "silu_mul", mul_operand=up_raw, dst=paired)
    torch.cuda.synchronize()
    assert np.array_equal(host(paired).view(np.uint32), a["q4_up_mul"].view(np.uint32))


@pytest.mark.parametrize("fmt,lim", [("f32", 95.0), ("q4b32", 130.0)])
def test_epilogue_extreme_accumulators(fmt, lim):
    """Identity W makes the accumulator equal x exactly; x sweeps [-lim, lim],
    through the range where e^-a overflows float32 (a < -88.7), so sigmoid and
    silu must be evaluated without overflow."""
    log(f"extreme accumulators {fmt} {lim}")
    N = K = 512
    x = np.linspace(-lim, lim, K).astype(np.float32)
    x[:4] = [-88.8, -89.5, 88.8, 89.5]
    if fmt == "f32":
        w = synth.Weights("f32", N, K, np.eye(N, K, dtype=np.float32).view(np.uint8).reshape(-1))
    else:
        codes = np.full((N, K), 8, dtype=np.uint8)
        np.fill_diagonal(codes, 9)
        w = synth.Weights("q4b32", N, K, synth.pack_q4b32(codes, np.ones((N, K // 32), np.float16)))
    m = synth.draw_vec(np.random.default_rng(5), N)
    for act in ("sigmoid", "silu", "silu_mul"):
        check_parity(w, x, act, m=m if act == "silu_mul" else None, tag=f"extreme {fmt} {act}")


def _identity_f32(n, scale=1.0):
    return synth.Weights("f32", n, n, (np.eye(n, dtype=np.float32) * np.float32(scale)).view(np.uint8).reshape(-1))


def _tail_sweep(n):
    """Accumulators through the range where e^a leaves float's normal range
    (a < -87.3) and silu(a) itself becomes subnormal (a < -95), to -130."""
    x = np.linspace(-130.0, 30.0, n).astype(np.float32)
    x[:6] = [-80.5, -87.5, -95.0, -103.4375, -103.9, -108.0]
    return x


def test_epilogue_tail_with_large_multiplier():
    """silu(a) * m with |m| = 40 for a in the float tail: the product is a
    float (down to the subnormals) although e^a alone is not, and it must
    still meet the oracle."""
    log("epilogue tail, large multiplier")
    N = 512
    w = _identity_f32(N)
    x = _tail_sweep(N)
    m = np.full(N, 40.0, np.float32)
    m[1::2] = -40.0
    for act in ("silu", "sigmoid", "silu_mul"):
        check_parity(w, x, act, m=m if act == "silu_mul" else None, tag=f"tail {act}")


def test_glu_tail_with_large_up():
    """The gated pair with gate sums through the float tail and up sums of
    40 times their size (identity matrices, the up one scaled by 40), one
    column and several; silu and sigmoid."""
    log("gated pair tail, large up")
    N = 512
    wg, wu = _identity_f32(N), _identity_f32(N, 40.0)
    x = _tail_sweep(N)
    for act in ("silu", "sigmoid"):
        check_glu(wg, wu, x, act, f"tail {act}")
        X = np.stack([x, x[::-1].copy(), -x])
        Wg, Wu, Xd = dev(wg.data), dev(wu.data), dev(X)
        dst = torch.full((3, N), float("nan"), dtype=torch.float32, device="cuda")
        binding.gemv_glu_ncols(Wg, Wu, "f32", N, N, 3, Xd, act, dst=dst)
        torch.cuda.synchronize()
        G = host(dst)
        Y, g, gA, u, uA = oracle.glu_ncols_reference("f32", N, N, wg.data, wu.data, X, act)
        from oracle.compare import compare_glu
        res = compare_glu(G.reshape(-1), Y.reshape(-1), act, g.reshape(-1), gA.reshape(-1), u.reshape(-1),
                          uA.reshape(-1))
        assert res["max_err"] <= TOLERANCE["f32"], (act, res)


# ------------------------------------------------------------------ gated pair (GLU)

def _glu(wg, wu, x, act, out_shape=None):
    Wg, Wu, xd = dev(wg.data), dev(wu.data), dev(x)
    dst = torch.full(out_shape or (wg.N,), float("nan"), dtype=torch.float32, device="cuda")
    binding.gemv_glu(Wg, Wu, wg.fmt, wg.N, wg.K, xd, act, dst=dst)
    torch.cuda.synchronize()
    return host(dst).reshape(-1)


def check_glu(wg, wu, x, act, tag):
    from oracle.compare import TOLERANCE, compare_glu
    log(f"glu {tag} fmt={wg.fmt} N={wg.N} K={wg.K} act={act}")
    g = _glu(wg, wu, x, act)
    y, ga, gA, ua, uA = oracle.glu_reference(wg.fmt, wg.N, wg.K, wg.data, wu.data, x, act)
    res = compare_glu(g, y, act, ga, gA, ua, uA)
    assert np.all(np.isfinite(g)), tag
    assert res["max_err"] <= TOLERANCE[wg.fmt], f"{tag}: {res}"
    assert_healthy(res, wg.fmt, wg.K, tag)
    return g


GLU_SHAPES = [(1, 32), (33, 96), (300, 512), (1003, 4096), (67, 14336), (17, 4128)]


@pytest.mark.parametrize("fmt", synth.FORMATS)
@pytest.mark.parametrize("N,K", GLU_SHAPES)
def test_glu_parity(fmt, N, K):
    rng = np.random.default_rng(zlib.crc32(f"glu/{fmt}/{N}/{K}".encode()))
    wg = synth.random_weights(rng, fmt, N, K)
    wu = synth.random_weights(rng, fmt, N, K)
    x = synth.draw_vec(rng, K)
    for act in ("silu", "sigmoid"):
        check_glu(wg, wu, x, act, f"{fmt} {N}x{K} {act}")


@pytest.mark.parametrize("fmt", ["f32", "f16"])
def test_glu_odd_k_generic_path(fmt):
    rng = np.random.default_rng(61)
    wg = synth.random_weights(rng, fmt, 40, 1001)
    wu = synth.random_weights(rng, fmt, 40, 1001)
    check_glu(wg, wu, synth.draw_vec(rng, 1001), "silu", f"{fmt} 40x1001")


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_glu_equals_composition_bitwise(fmt):
    """gemv_glu(W_g, W_u) == gemv_fused(W_u, none) then gemv_fused(W_g, silu_mul, m = up), bit for bit."""
    log(f"glu == composition {fmt}")
    rng = np.random.default_rng(62)
    N, K = 2050, 4096
    wg = synth.random_weights(rng, fmt, N, K)
    wu = synth.random_weights(rng, fmt, N, K)
    x = synth.draw_vec(rng, K)
    Wg, Wu, xd = dev(wg.data), dev(wu.data), dev(x)
    up = torch.empty(N, dtype=torch.float32, device="cuda")
    comp = torch.empty(N, dtype=torch.float32, device="cuda")
    binding.gemv_fused(Wu, fmt, N, K, xd, "none", dst=up)
    binding.gemv_fused(Wg, fmt, N, K, xd, "silu_mul", mul_operand=up, dst=comp)
    fused = torch.empty(N, dtype=torch.float32, device="cuda")
    binding.gemv_glu(Wg, Wu, fmt, N, K, xd, "silu", dst=fused)
    torch.cuda.synchronize()
    assert np.array_equal(host(fused).view(np.uint32), host(comp).view(np.uint32))


def test_glu_full_size_layer_gate_up():
    """The 4-bit layer's gate and up projections (14336 x 4096) as one gated pair."""
    wl = synth.q4b32_decode_layer(0)
    check_glu(wl.weights["Wgate"], wl.weights["Wup"], wl.vectors["x_ffn"], "silu", "q4 layer gate/up 14336x4096")


def test_glu_rejected_writes_nothing():
    rng = np.random.default_rng(63)
    w = synth.random_weights(rng, "f16", 64, 64)
    Wd, xd = dev(w.data), dev(synth.draw_vec(rng, 64))
    dst = torch.full((64,), 3.0, dtype=torch.float32, device="cuda")
    with pytest.raises(binding.GemvError) as e:
        binding.gemv_glu(Wd, Wd, "f16", 64, 64, xd, "add", dst=dst)
    assert e.value.status == binding.STATUS_CODE["GEMV_E_ACT"]
    torch.cuda.synchronize()
    assert torch.all(dst == 3.0)


# ------------------------------------------------------------------ shape-chosen wave counts

@pytest.mark.parametrize("fmt,N,K", [("f16", 4096, 14336), ("bf16", 4096, 6144), ("f32", 4096, 4096),
                                     ("f16", 4096, 4096), ("bf16", 2048, 14336), ("f16", 4095, 4096)])
def test_wave_count_paths(fmt, N, K):
    """Shapes that take the 16- and 8-wave workgroups (long rows; rows that
    fill one 16-wave workgroup per CU) against the oracle, and fused ==
    unfused bit for bit on them."""
    rng = np.random.default_rng(N + K)
    w = synth.random_weights(rng, fmt, N, K)
    x = synth.draw_vec(rng, K)
    r = rng.normal(size=N).astype(np.float32)
    check_parity(w, x, "add", r=r, tag=f"waves {N}x{K}")
    f, u = _fused_and_unfused(w, x, "silu_mul", rng.normal(size=N).astype(np.float32), None)
    assert np.array_equal(f.view(np.uint32), u.view(np.uint32))
