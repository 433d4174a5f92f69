"""The C ABI on the host, with no GPU: the library loads, exports every
function the header declares, and its checks return the documented status for
every invalid-argument path.  Pointers here are plain integers; gemv_validate
never dereferences them and makes no HIP call."""
import os
import re

import pytest

import oracle
from decode_gemv_elementwise_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
S = b.STATUS_CODE

W0 = 1 << 20            # fake device addresses, far apart
X0 = 1 << 30
D0 = 1 << 34
M0 = 1 << 36
R0 = 1 << 38


def declared_functions():
    text = open(os.path.join(ROOT, "include", "gemv_fused.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = b.load()
    names = declared_functions()
    assert {"gemv_fused", "gemv_validate", "gemv_epilogue", "gemv_epilogue_validate", "gemv_weight_bytes",
            "gemv_strerror", "gemv_last_hip_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_probe_library_exports_every_declared_function():
    import ctypes
    from decode_gemv_elementwise_amd import build as bld
    text = open(os.path.join(ROOT, "include", "hbm_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b((?:hbm|gemv)_[a-z_]+)\s*\(", text)))
    assert {"hbm_read_probe", "hbm_read_once", "hbm_read_once_blocks", "hbm_read_floor", "hbm_read_floor_shapes",
            "hbm_read_floor_out_floats", "gemv_valu_floor", "hbm_copy"} <= set(names)
    lib = ctypes.CDLL(bld.PROBE_LIB)
    for n in names:
        assert hasattr(lib, n), n
    lib.hbm_read_once_blocks.argtypes = [ctypes.c_int64]
    assert lib.hbm_read_once_blocks(16) == 1
    assert lib.hbm_read_once_blocks(32768) == 1 and lib.hbm_read_once_blocks(32784) == 2
    assert lib.hbm_read_once_blocks(0) == -1


def test_status_strings():
    for code in S.values():
        assert b.gemv_strerror(code)
    assert b.gemv_strerror(123) == "unknown status"
    assert b.gemv_last_hip_error() == 0


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16", "q8b32", "q4b32"])
@pytest.mark.parametrize("N,K", [(1, 32), (4096, 4096), (14336, 4096), (4096, 14336), (3, 64), (32, 4096)])
def test_weight_bytes_agrees_with_oracle(fmt, N, K):
    assert b.gemv_weight_bytes(fmt, N, K) == oracle.weight_bytes(fmt, N, K)


def test_weight_bytes_errors():
    assert b.gemv_weight_bytes("q4b32", 4, 33) == S["GEMV_E_DIM"]
    assert b.gemv_weight_bytes("f32", 0, 4) == S["GEMV_E_DIM"]
    assert b.gemv_weight_bytes(7, 4, 4) == S["GEMV_E_FMT"]
    assert b.gemv_weight_bytes("f32", 1 << 31, 4) == S["GEMV_E_DIM"]
    # both extents legal, but four bytes per weight no longer fit in int64
    big = (1 << 31) - 1
    assert b.gemv_weight_bytes("f32", big, big) == S["GEMV_E_DIM"]
    assert b.gemv_weight_bytes("f16", big, big) == 2 * big * big


def v(addr, shape, stride=None):
    return b.make_view(addr, shape, stride)


def val(**kw):
    args = dict(W=W0, wfmt="f32", N=64, K=64, x=X0, act="none", mul_operand=None, add_operand=None,
                dst=v(D0, (64,)))
    args.update(kw)
    return b.gemv_validate(args["W"], args["wfmt"], args["N"], args["K"], args["x"], args["act"],
                           args["mul_operand"], args["add_operand"], args["dst"])


def test_valid_calls():
    assert val() == S["GEMV_OK"]
    for act in ("sigmoid", "silu"):
        assert val(act=act) == S["GEMV_OK"]
    assert val(act="silu_mul", mul_operand=v(M0, (64,))) == S["GEMV_OK"]
    assert val(act="mul", mul_operand=v(M0, (64,))) == S["GEMV_OK"]
    assert val(act="add", add_operand=v(R0, (64,))) == S["GEMV_OK"]
    # the [32, 128] view of a 4096-row output, residual of the same shape
    assert val(N=4096, K=6144, wfmt="q8b32", act="add", add_operand=v(R0, (32, 128)),
               dst=v(D0, (32, 128))) == S["GEMV_OK"]
    # in place: dst is the identical view of the operand
    assert val(act="add", add_operand=v(R0, (64,)), dst=v(R0, (64,))) == S["GEMV_OK"]
    assert val(act="mul", mul_operand=v(M0, (8, 8)), dst=v(M0, (8, 8))) == S["GEMV_OK"]
    # extent-1 dimensions may carry any stride
    assert val(dst=v(D0, (1, 64), (999, 1))) == S["GEMV_OK"]
    # float formats accept any K
    assert val(K=7) == S["GEMV_OK"]
    assert val(wfmt="f16", K=1) == S["GEMV_OK"]
    # read-only inputs may overlap each other (x inside W here)
    assert val(x=W0 + 64) == S["GEMV_OK"]


def test_null_pointers():
    assert val(W=0) == S["GEMV_E_NULL"]
    assert val(x=0) == S["GEMV_E_NULL"]
    assert val(dst=None) == S["GEMV_E_NULL"]
    assert val(dst=v(0, (64,))) == S["GEMV_E_NULL"]
    assert val(act="add", add_operand=v(0, (64,))) == S["GEMV_E_NULL"]


def test_format_and_act():
    assert val(wfmt=5) == S["GEMV_E_FMT"]
    assert val(wfmt=-1) == S["GEMV_E_FMT"]
    assert val(act=6) == S["GEMV_E_ACT"]
    assert val(act=-1) == S["GEMV_E_ACT"]


def test_dimensions():
    assert val(N=0, dst=v(D0, (0,))) == S["GEMV_E_DIM"]
    assert val(K=0) == S["GEMV_E_DIM"]
    assert val(K=-5) == S["GEMV_E_DIM"]
    assert val(wfmt="q4b32", K=48) == S["GEMV_E_DIM"]
    assert val(wfmt="q8b32", K=16) == S["GEMV_E_DIM"]
    assert val(N=65, dst=v(D0, (64,))) == S["GEMV_E_DIM"]          # dst holds 64 != N
    assert val(dst=v(D0, (8, 9))) == S["GEMV_E_DIM"]
    assert val(K=1 << 31) == S["GEMV_E_DIM"]


def test_operand_presence():
    assert val(act="add") == S["GEMV_E_OPERAND"]
    assert val(act="mul") == S["GEMV_E_OPERAND"]
    assert val(act="silu_mul") == S["GEMV_E_OPERAND"]
    assert val(act="none", add_operand=v(R0, (64,))) == S["GEMV_E_OPERAND"]
    assert val(act="sigmoid", mul_operand=v(M0, (64,))) == S["GEMV_E_OPERAND"]
    assert val(act="add", add_operand=v(R0, (64,)), mul_operand=v(M0, (64,))) == S["GEMV_E_OPERAND"]
    assert val(act="mul", add_operand=v(R0, (64,))) == S["GEMV_E_OPERAND"]


def test_layout():
    assert val(dst=v(D0, (64,), (2,))) == S["GEMV_E_LAYOUT"]                      # strided
    assert val(dst=v(D0, (8, 8), (1, 8))) == S["GEMV_E_LAYOUT"]                   # transposed
    assert val(dst=v(D0, (1, 1, 1, 1, 64))) == S["GEMV_E_LAYOUT"]                 # rank 5
    assert val(act="add", add_operand=v(R0, (8, 8)), dst=v(D0, (64,))) == S["GEMV_E_LAYOUT"]  # shape differs
    assert val(act="add", add_operand=v(R0, (1, 64)), dst=v(D0, (64,))) == S["GEMV_E_LAYOUT"]  # no broadcast
    assert val(act="add", add_operand=v(R0, (64,), (2,))) == S["GEMV_E_LAYOUT"]
    assert val(dst=v(D0, (-64,))) == S["GEMV_E_LAYOUT"]


def test_alignment():
    assert val(W=W0 + 4) == S["GEMV_E_ALIGN"]
    assert val(x=X0 + 2) == S["GEMV_E_ALIGN"]
    assert val(dst=v(D0 + 1, (64,))) == S["GEMV_E_ALIGN"]
    assert val(act="add", add_operand=v(R0 + 2, (64,))) == S["GEMV_E_ALIGN"]


def test_alias_rules():
    wbytes = 64 * 64 * 4
    assert val(dst=v(W0, (64,))) == S["GEMV_E_ALIAS"]                       # dst on W
    assert val(dst=v(W0 + wbytes - 4, (64,))) == S["GEMV_E_ALIAS"]          # last byte of W
    assert val(dst=v(W0 + wbytes, (64,))) == S["GEMV_OK"]                   # just past W
    assert val(dst=v(X0 - 252, (64,))) == S["GEMV_E_ALIAS"]                 # dst tail on x
    assert val(dst=v(X0 - 256, (64,))) == S["GEMV_OK"]                      # touches, no overlap
    assert val(dst=v(X0 + 64 * 4, (64,))) == S["GEMV_OK"]
    # partial overlap with the operand is refused, identity is allowed
    assert val(act="add", add_operand=v(R0, (64,)), dst=v(R0 + 4, (64,))) == S["GEMV_E_ALIAS"]
    assert val(act="add", add_operand=v(R0 + 4, (64,)), dst=v(R0, (64,))) == S["GEMV_E_ALIAS"]
    assert val(act="mul", mul_operand=v(M0, (64,)), dst=v(M0 + 252, (64,))) == S["GEMV_E_ALIAS"]
    # the check is stateless: a refused call does not change the next verdict
    assert val(act="add", add_operand=v(R0, (64,)), dst=v(R0, (64,))) == S["GEMV_OK"]
    # a buffer running past the top of the address space is no buffer: it
    # counts as overlapping everything (dst lies in what a wrapped span of W
    # would otherwise have reached from address 0)
    top = (1 << 64) - 256
    assert val(W=top, dst=v(256, (64,))) == S["GEMV_E_ALIAS"]
    assert val(x=top + 128, dst=v(256, (64,))) == S["GEMV_E_ALIAS"]
    assert val(dst=v(top + 192, (64,))) == S["GEMV_E_ALIAS"]
    assert val(W=top - wbytes, dst=v(256, (64,))) == S["GEMV_OK"]          # ends just below the top


def eval_(act="none", N=64, acc=X0, mul=None, add=None, dst=None):
    return b.gemv_epilogue_validate(act, N, acc, mul, add, dst if dst is not None else v(D0, (N,)))


def test_epilogue_validate():
    assert eval_() == S["GEMV_OK"]
    assert eval_(act="add", add=v(R0, (64,))) == S["GEMV_OK"]
    assert eval_(act="add", add=v(R0, (64,)), dst=v(X0, (64,))) == S["GEMV_OK"]   # in place on acc
    assert eval_(act="add", add=v(R0, (64,)), dst=v(R0, (64,))) == S["GEMV_OK"]   # in place on r
    assert eval_(act="add", add=v(R0, (64,)), dst=v(X0 + 4, (64,))) == S["GEMV_E_ALIAS"]
    assert eval_(act="add") == S["GEMV_E_OPERAND"]
    assert eval_(acc=0) == S["GEMV_E_NULL"]
    assert eval_(N=0, dst=v(D0, (0,))) == S["GEMV_E_DIM"]
    assert eval_(act=17) == S["GEMV_E_ACT"]
    assert eval_(acc=X0 + 1) == S["GEMV_E_ALIGN"]


U0 = 1 << 24  # a second fake weight matrix


def gval(**kw):
    args = dict(Wg=W0, Wu=U0, wfmt="f16", N=64, K=64, x=X0, act="silu", dst=v(D0, (64,)))
    args.update(kw)
    return b.gemv_glu_validate(args["Wg"], args["Wu"], args["wfmt"], args["N"], args["K"], args["x"], args["act"],
                               args["dst"])


def test_glu_validate():
    assert gval() == S["GEMV_OK"]
    assert gval(act="sigmoid") == S["GEMV_OK"]
    assert gval(Wu=W0) == S["GEMV_OK"]                       # the same matrix twice is allowed
    assert gval(dst=v(D0, (8, 8))) == S["GEMV_OK"]
    for act in ("none", "silu_mul", "mul", "add", 9):
        assert gval(act=act) == S["GEMV_E_ACT"]
    assert gval(Wg=0) == S["GEMV_E_NULL"]
    assert gval(Wu=0) == S["GEMV_E_NULL"]
    assert gval(dst=None) == S["GEMV_E_NULL"]
    assert gval(wfmt=5) == S["GEMV_E_FMT"]
    assert gval(wfmt="q4b32", K=48) == S["GEMV_E_DIM"]
    assert gval(N=65) == S["GEMV_E_DIM"]
    assert gval(dst=v(D0, (64,), (2,))) == S["GEMV_E_LAYOUT"]
    assert gval(Wu=U0 + 8) == S["GEMV_E_ALIGN"]
    assert gval(dst=v(U0 + 64, (64,))) == S["GEMV_E_ALIAS"]   # dst on the up matrix
    assert gval(dst=v(W0, (64,))) == S["GEMV_E_ALIAS"]        # dst on the gate matrix
    assert gval(dst=v(X0, (64,))) == S["GEMV_E_ALIAS"]        # dst on x


def gnval(ncols=4, **kw):
    args = dict(Wg=W0, Wu=U0, wfmt="f16", N=64, K=64, x=X0, act="silu", dst=v(D0, (ncols, 64)))
    args.update(kw)
    return b.gemv_glu_ncols_validate(args["Wg"], args["Wu"], args["wfmt"], args["N"], args["K"], ncols,
                                     args["x"], args["act"], args["dst"])


def test_glu_ncols_validate():
    assert gnval() == S["GEMV_OK"]
    assert gnval(ncols=8, dst=v(D0, (8 * 64,))) == S["GEMV_OK"]
    assert gnval(ncols=1, dst=v(D0, (64,))) == S["GEMV_OK"]
    assert gnval(act="sigmoid") == S["GEMV_OK"]
    for nc in (0, 9, -1):
        assert gnval(ncols=nc, dst=v(D0, (64,))) == S["GEMV_E_DIM"]
    assert gnval(dst=v(D0, (3, 64))) == S["GEMV_E_DIM"]                # dst holds 3 columns, not 4
    for act in ("none", "silu_mul", "mul", "add"):
        assert gnval(act=act) == S["GEMV_E_ACT"]
    assert gnval(Wu=0) == S["GEMV_E_NULL"]
    assert gnval(wfmt="q8b32", K=48) == S["GEMV_E_DIM"]
    assert gnval(x=X0 + 2) == S["GEMV_E_ALIGN"]
    # dst may not reach into any column of x, nor into either matrix
    assert gnval(dst=v(X0 + 3 * 64 * 4, (4, 64))) == S["GEMV_E_ALIAS"]  # on x's fourth column
    assert gnval(dst=v(X0 + 4 * 64 * 4, (4, 64))) == S["GEMV_OK"]       # just past x
    assert gnval(dst=v(U0 + 64, (4, 64))) == S["GEMV_E_ALIAS"]
    # one column is the one-column pair's check
    for kw in (dict(), dict(act="none"), dict(Wu=U0 + 8), dict(dst=v(U0, (64,)))):
        dst = kw.pop("dst", v(D0, (64,)))
        a = gnval(ncols=1, dst=dst, **kw)
        g = gval(dst=dst, **kw)
        assert a == g, kw


def nval(ncols=4, **kw):
    args = dict(W=W0, wfmt="f16", N=64, K=64, x=X0, act="none", mul_operand=None, add_operand=None,
                dst=v(D0, (ncols, 64)))
    args.update(kw)
    return b.gemv_fused_ncols_validate(args["W"], args["wfmt"], args["N"], args["K"], ncols, args["x"],
                                       args["act"], args["mul_operand"], args["add_operand"], args["dst"])


def test_ncols_validate():
    for n in range(1, 9):
        assert nval(ncols=n) == S["GEMV_OK"]
    assert nval(ncols=0, dst=v(D0, (1, 64))) == S["GEMV_E_DIM"]
    assert nval(ncols=9, dst=v(D0, (9, 64))) == S["GEMV_E_DIM"]
    assert nval(ncols=-1, dst=v(D0, (64,))) == S["GEMV_E_DIM"]
    # dst must hold ncols * N elements, in any C-contiguous shape
    assert nval(dst=v(D0, (256,))) == S["GEMV_OK"]
    assert nval(dst=v(D0, (4, 2, 32))) == S["GEMV_OK"]
    assert nval(dst=v(D0, (64,))) == S["GEMV_E_DIM"]
    assert nval(dst=v(D0, (4, 64), (1, 4))) == S["GEMV_E_LAYOUT"]
    # operands have dst's shape
    assert nval(act="add", add_operand=v(R0, (4, 64))) == S["GEMV_OK"]
    assert nval(act="add", add_operand=v(R0, (64,))) == S["GEMV_E_LAYOUT"]
    assert nval(act="silu_mul", mul_operand=v(M0, (4, 64)), dst=v(M0, (4, 64))) == S["GEMV_OK"]
    assert nval(act="silu_mul") == S["GEMV_E_OPERAND"]
    # x spans ncols * K floats: dst right after one column of x still overlaps
    assert nval(dst=v(X0 + 64 * 4, (4, 64))) == S["GEMV_E_ALIAS"]
    assert nval(ncols=1, dst=v(X0 + 64 * 4, (1, 64))) == S["GEMV_OK"]
    # partial overlap with the operand
    assert nval(act="add", add_operand=v(R0, (4, 64)), dst=v(R0 + 4, (4, 64))) == S["GEMV_E_ALIAS"]
    assert nval(wfmt="q4b32", K=48) == S["GEMV_E_DIM"]
    assert nval(W=0) == S["GEMV_E_NULL"]
    assert nval(act=6) == S["GEMV_E_ACT"]


def test_ncols_one_column_matches_gemv_validate():
    cases = [dict(), dict(act="add", add_operand=v(R0, (64,))), dict(dst=v(X0, (64,))), dict(K=7),
             dict(wfmt="q8b32", K=40), dict(dst=v(D0, (63,)))]
    for kw in cases:
        d = dict(wfmt="f32", dst=v(D0, (64,)))
        d.update(kw)
        assert nval(ncols=1, **d) == val(**d), kw


def fval(**kw):
    args = dict(x=X0, signs=M0, nrows=2, K=4096, n=1024, nsigns=4096, dst=D0)
    args.update(kw)
    return b.gemv_fwht_signed_validate(args["x"], args["signs"], args["nrows"], args["K"], args["n"],
                                       args["nsigns"], args["dst"])


def test_fwht_validate():
    assert fval() == S["GEMV_OK"]
    for n in (1, 2, 64, 512, 1024):
        assert fval(n=n) == S["GEMV_OK"]
    assert fval(n=2048, K=4096) == S["GEMV_E_DIM"]          # beyond one wave's tile
    assert fval(n=3) == S["GEMV_E_DIM"]                     # not a power of two
    assert fval(n=0) == S["GEMV_E_DIM"]
    assert fval(K=1536, n=1024, nsigns=512) == S["GEMV_E_DIM"]   # n does not divide K
    assert fval(nsigns=3) == S["GEMV_E_DIM"]                # nsigns does not divide K
    assert fval(nsigns=1) == S["GEMV_OK"]
    assert fval(nrows=0) == S["GEMV_E_DIM"]
    assert fval(nrows=1 << 20, K=4096) == S["GEMV_E_DIM"]   # nrows * K too large
    assert fval(nrows=(1 << 63) - 1, K=4096) == S["GEMV_E_DIM"]   # no overflow in nrows * K
    assert fval(x=0) == S["GEMV_E_NULL"] and fval(signs=0) == S["GEMV_E_NULL"] and fval(dst=0) == S["GEMV_E_NULL"]
    assert fval(x=X0 + 2) == S["GEMV_E_ALIGN"] and fval(signs=M0 + 1) == S["GEMV_E_ALIGN"]
    assert fval(dst=X0) == S["GEMV_OK"]                     # in place
    assert fval(dst=X0 + 4) == S["GEMV_E_ALIAS"]            # shifted overlap
    assert fval(dst=M0) == S["GEMV_E_ALIAS"]                # over the signs
    assert fval(x=X0 + 4, dst=X0 + 4, K=7, n=1, nsigns=7) == S["GEMV_OK"]   # any K for n = 1


def ffval(**kw):
    args = dict(W=W0, wfmt="f16", N=64, K=4096, x=X0, signs=M0, n=1024, nsigns=4096, act="add",
                mul_operand=None, add_operand=v(R0, (64,)), dst=v(D0, (64,)))
    args.update(kw)
    return b.gemv_fused_fwht_validate(args["W"], args["wfmt"], args["N"], args["K"], args["x"], args["signs"],
                                      args["n"], args["nsigns"], args["act"], args["mul_operand"],
                                      args["add_operand"], args["dst"])


def test_fused_fwht_validate():
    assert ffval() == S["GEMV_OK"]
    assert ffval(wfmt="q4b32", K=14336, nsigns=1024) == S["GEMV_OK"]
    assert ffval(signs=0) == S["GEMV_E_NULL"]
    assert ffval(n=2048) == S["GEMV_E_DIM"]
    assert ffval(nsigns=3) == S["GEMV_E_DIM"]
    # only the chunked kernel carries the transform: whole 16-byte chunks, x within LDS
    assert ffval(wfmt="f16", K=4100, n=4, nsigns=4) == S["GEMV_E_DIM"]
    assert ffval(wfmt="f32", K=4100, n=4, nsigns=4) == S["GEMV_OK"]
    assert ffval(wfmt="f16", K=32768, nsigns=1) == S["GEMV_E_DIM"]
    assert ffval(wfmt="q4b32", K=32768, nsigns=1) == S["GEMV_OK"]
    assert ffval(dst=v(M0, (64,))) == S["GEMV_E_ALIAS"]      # dst over the signs
    assert ffval(signs=M0 + 2) == S["GEMV_E_ALIGN"]
    # the gemv_fused checks come first
    assert ffval(act="add", add_operand=None) == S["GEMV_E_OPERAND"]
    assert ffval(dst=v(X0, (64,))) == S["GEMV_E_ALIAS"]


def test_ncols_kernel_query_arguments():
    """The query needs no device for rejected arguments or one column."""
    assert b.gemv_ncols_kernel("f16", 64, 64, 1) == "one_column"
    assert b.gemv_ncols_kernel("q4b32", 4096, 4096, 1) == "one_column"
    for args, code in [(("f16", 0, 64, 2), "GEMV_E_DIM"), (("f16", 64, 0, 2), "GEMV_E_DIM"),
                       (("f16", 64, 64, 9), "GEMV_E_DIM"), (("f16", 64, 64, 0), "GEMV_E_DIM"),
                       (("q8b32", 64, 48, 2), "GEMV_E_DIM"), (("q4b32", 64, 1 << 31, 2), "GEMV_E_DIM")]:
        with pytest.raises(b.GemvError) as e:
            b.gemv_ncols_kernel(*args)
        assert e.value.status == S[code], args
    assert b.load().gemv_ncols_kernel(9, 64, 64, 2) == S["GEMV_E_FMT"]
