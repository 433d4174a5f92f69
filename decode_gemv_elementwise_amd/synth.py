"""Seeded synthetic inputs for the fused decode GEMV, and the weight packers.

This module only draws random numbers and lays them out in the storage
formats; it holds none of the product's arithmetic, and both the GPU tests and
the CPU oracle consume what it makes.  numpy only.

Workloads (the decode shapes of a dense 4096-hidden / 14336-FFN layer):

* ``f32_tiny_256``: W 256x256 f32 ~N(0, 1/256) (variance 1/256, std 1/16);
  x, m, r 256 f32 ~N(0,1); every epilogue.
* ``f16_outproj_residual_4096``: W 4096x4096 f16 ~N(0, 1/4096); x 4096;
  residual r 4096; dst = W x + r with dst aliasing r in place.
* ``bf16_swiglu_gate_14336x4096``: W 14336x4096 bf16 ~N(0, 1/4096); x 4096;
  m 14336; dst = silu(W x) * m; plus a 32x4096 bf16 sigmoid gate on the same x.
* ``q8b32_view_residual_4096x6144``: 8-bit block weights 4096x6144 (codes
  ~U{-127..127}, one fp16 scale ~U(0.001, 0.01) per 32 codes); x 6144;
  output viewed as [32, 128] plus a contiguous [32, 128] residual.
* ``q4b32_decode_layer``: six 4-bit block GEMVs of one decode layer (codes
  ~U{0..15}, scale ~U(0.001, 0.02), value = (code - 8) * scale):
  4096->6144 none, 4096->4096 +residual, 4096->14336 silu (gate),
  4096->14336 * gate output (up), 14336->4096 +residual (down, input = the up
  output), 4096->32 sigmoid.
* ``q4b32_decode_layer_glu``: the same layer with gate and up as one gated
  pair, silu(W_gate x) * (W_up x) (five calls).
* ``f16_outproj_fwht_residual_4096``: the f16 residual projection after the
  signed Hadamard transform of x (blocks of 1024, signs +-1 drawn uniformly).
* ``f16_outproj_residual_4096_ncols8``, ``q4b32_gate_14336x4096_ncols4``:
  several destination columns over one W (x [ncols, K], operands and dst
  [ncols, N]).

Draw order per workload, one ``numpy.random.default_rng(seed)`` each: weights
(codes, then scales) in call order, then x, then m, then r.  Floats are drawn
in float64 and rounded to nearest-even into the storage type; the stored value
is the truth both sides consume.
"""
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

FORMATS = ("f32", "f16", "bf16", "q8b32", "q4b32")
ACTS = ("none", "sigmoid", "silu", "silu_mul", "mul", "add")


def align256(v: int) -> int:
    return (v + 255) // 256 * 256


# ---------------------------------------------------------------- packers

def bf16_bits_from_f32(a) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest-even) and return the bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def pack_q8b32(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes int8 [N, K], scales float16 [N, K/32] -> bytes: the int8 codes
    plane (row-major), then the fp16 scales plane at the next 256-byte
    boundary."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    N, K = codes.shape
    assert K % 32 == 0 and scales.shape == (N, K // 32)
    off = align256(N * K)
    out = np.zeros(off + N * (K // 32) * 2, dtype=np.uint8)
    out[: N * K] = codes.view(np.uint8).reshape(-1)
    out[off:] = np.ascontiguousarray(scales, dtype="<f2").view(np.uint8).reshape(-1)
    return out


def pack_q4b32(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes uint8 in 0..15 [N, K], scales float16 [N, K/32] -> bytes: the
    nibble plane (byte k/2 of a row holds element k in its low nibble when k
    is even, in its high nibble when k is odd), then the fp16 scales plane at
    the next 256-byte boundary."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    N, K = codes.shape
    assert K % 32 == 0 and scales.shape == (N, K // 32)
    assert int(codes.max(initial=0)) < 16
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    off = align256(N * K // 2)
    out = np.zeros(off + N * (K // 32) * 2, dtype=np.uint8)
    out[: N * K // 2] = packed.reshape(-1)
    out[off:] = np.ascontiguousarray(scales, dtype="<f2").view(np.uint8).reshape(-1)
    return out


def weight_nbytes(fmt: str, N: int, K: int) -> int:
    if fmt == "f32":
        return N * K * 4
    if fmt in ("f16", "bf16"):
        return N * K * 2
    if fmt == "q8b32":
        return align256(N * K) + N * (K // 32) * 2
    if fmt == "q4b32":
        return align256(N * K // 2) + N * (K // 32) * 2
    raise ValueError(fmt)


# ---------------------------------------------------------------- draws

@dataclass
class Weights:
    fmt: str
    N: int
    K: int
    data: np.ndarray  # uint8 byte image in the storage format
    # pre-packing parts, for tests that need them
    codes: Optional[np.ndarray] = None
    scales: Optional[np.ndarray] = None


def draw_float_weights(rng, fmt: str, N: int, K: int, var: float) -> Weights:
    v = rng.normal(0.0, np.sqrt(var), size=(N, K))
    if fmt == "f32":
        data = v.astype(np.float32)
    elif fmt == "f16":
        data = v.astype(np.float16)
    elif fmt == "bf16":
        data = bf16_bits_from_f32(v.astype(np.float32)).reshape(N, K)
    else:
        raise ValueError(fmt)
    return Weights(fmt, N, K, np.ascontiguousarray(data).view(np.uint8).reshape(-1))


def draw_q8b32(rng, N: int, K: int, scale_lo: float, scale_hi: float) -> Weights:
    codes = rng.integers(-127, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    scales = rng.uniform(scale_lo, scale_hi, size=(N, K // 32)).astype(np.float16)
    return Weights("q8b32", N, K, pack_q8b32(codes, scales), codes, scales)


def draw_q4b32(rng, N: int, K: int, scale_lo: float, scale_hi: float) -> Weights:
    codes = rng.integers(0, 16, size=(N, K), dtype=np.int64).astype(np.uint8)
    scales = rng.uniform(scale_lo, scale_hi, size=(N, K // 32)).astype(np.float16)
    return Weights("q4b32", N, K, pack_q4b32(codes, scales), codes, scales)


def draw_vec(rng, n: int) -> np.ndarray:
    return rng.normal(0.0, 1.0, size=n).astype(np.float32)


# ---------------------------------------------------------------- workloads

@dataclass
class Call:
    """One fused GEMV call.  ``w``, ``x``, ``m``, ``r`` name entries of the
    workload's tensors, or the output of an earlier call ("@name")."""
    name: str
    w: str
    x: str
    act: str
    m: Optional[str] = None
    r: Optional[str] = None
    out_shape: Optional[Tuple[int, ...]] = None  # view shape of dst (default [N])
    inplace: bool = False  # dst is the same memory as the add/mul operand
    w2: Optional[str] = None  # up matrix of a gated pair: dst = act(w x) * (w2 x)
    ncols: int = 1  # destination columns: x is [ncols, K], dst and operands [ncols, N]
    fwht: Optional[Tuple[str, int]] = None  # (signs, n): x goes through the signed Hadamard transform first


@dataclass
class Workload:
    name: str
    weights: Dict[str, Weights]
    vectors: Dict[str, np.ndarray]
    calls: List[Call] = field(default_factory=list)
    description: str = ""


def f32_tiny_256(seed: int = 0) -> Workload:
    rng = np.random.default_rng(seed)
    W = draw_float_weights(rng, "f32", 256, 256, 1.0 / 256)
    x, m, r = draw_vec(rng, 256), draw_vec(rng, 256), draw_vec(rng, 256)
    calls = [Call(f"f32_256_{a}", "W", "x", a,
                  m="m" if a in ("silu_mul", "mul") else None,
                  r="r" if a == "add" else None) for a in ACTS]
    return Workload("f32_tiny_256", {"W": W}, {"x": x, "m": m, "r": r}, calls,
                    "W 256x256 f32 ~N(0,1/256); x, m, r ~N(0,1); every epilogue")


def f16_outproj_residual_4096(seed: int = 0) -> Workload:
    rng = np.random.default_rng(seed)
    W = draw_float_weights(rng, "f16", 4096, 4096, 1.0 / 4096)
    x, r = draw_vec(rng, 4096), draw_vec(rng, 4096)
    calls = [Call("f16_outproj_add_inplace", "W", "x", "add", r="r", inplace=True)]
    return Workload("f16_outproj_residual_4096", {"W": W}, {"x": x, "r": r}, calls,
                    "W 4096x4096 f16 ~N(0,1/4096); dst = W x + r, dst aliasing r")


def bf16_swiglu_gate_14336x4096(seed: int = 0) -> Workload:
    rng = np.random.default_rng(seed)
    W = draw_float_weights(rng, "bf16", 14336, 4096, 1.0 / 4096)
    x, m = draw_vec(rng, 4096), draw_vec(rng, 14336)
    Wg = draw_float_weights(rng, "bf16", 32, 4096, 1.0 / 4096)
    calls = [Call("bf16_swiglu_silu_mul", "W", "x", "silu_mul", m="m"),
             Call("bf16_gate_sigmoid_32", "Wg", "x", "sigmoid")]
    return Workload("bf16_swiglu_gate_14336x4096", {"W": W, "Wg": Wg}, {"x": x, "m": m}, calls,
                    "W 14336x4096 bf16 ~N(0,1/4096); dst = silu(W x) * m; 32x4096 sigmoid gate")


def q8b32_view_residual_4096x6144(seed: int = 0) -> Workload:
    rng = np.random.default_rng(seed)
    W = draw_q8b32(rng, 4096, 6144, 0.001, 0.01)
    x = draw_vec(rng, 6144)
    r = draw_vec(rng, 4096).reshape(32, 128)
    calls = [Call("q8b32_add_view_32x128", "W", "x", "add", r="r", out_shape=(32, 128))]
    return Workload("q8b32_view_residual_4096x6144", {"W": W}, {"x": x, "r": r}, calls,
                    "8-bit blocks 4096x6144; output viewed [32,128] + residual [32,128]")


def q4b32_decode_layer(seed: int = 0) -> Workload:
    rng = np.random.default_rng(seed)
    shapes = [("Wqkv", 6144, 4096), ("Wo", 4096, 4096), ("Wgate", 14336, 4096),
              ("Wup", 14336, 4096), ("Wdown", 4096, 14336), ("Wg", 32, 4096)]
    weights = {n: draw_q4b32(rng, N, K, 0.001, 0.02) for n, N, K in shapes}
    vectors = {"x_qkv": draw_vec(rng, 4096), "x_o": draw_vec(rng, 4096),
               "x_ffn": draw_vec(rng, 4096), "x_g": draw_vec(rng, 4096),
               "r_o": draw_vec(rng, 4096), "r_down": draw_vec(rng, 4096)}
    calls = [Call("q4_qkv_none", "Wqkv", "x_qkv", "none"),
             Call("q4_o_add", "Wo", "x_o", "add", r="r_o"),
             Call("q4_gate_silu", "Wgate", "x_ffn", "silu"),
             Call("q4_up_mul", "Wup", "x_ffn", "mul", m="@q4_gate_silu"),
             Call("q4_down_add", "Wdown", "@q4_up_mul", "add", r="r_down"),
             Call("q4_gate_sigmoid_32", "Wg", "x_g", "sigmoid")]
    return Workload("q4b32_decode_layer", weights, vectors, calls,
                    "six 4-bit block GEMVs of one decode layer, chained gate -> up -> down")


def q4b32_decode_layer_glu(seed: int = 0) -> Workload:
    """The same draws as q4b32_decode_layer, with the gate and up projections
    issued as one gated pair (silu(W_gate x) * (W_up x)): five calls."""
    wl = q4b32_decode_layer(seed)
    calls = [Call("q4_qkv_none", "Wqkv", "x_qkv", "none"),
             Call("q4_o_add", "Wo", "x_o", "add", r="r_o"),
             Call("q4_gate_up_glu", "Wgate", "x_ffn", "silu", w2="Wup"),
             Call("q4_down_add", "Wdown", "@q4_gate_up_glu", "add", r="r_down"),
             Call("q4_gate_sigmoid_32", "Wg", "x_g", "sigmoid")]
    return Workload("q4b32_decode_layer_glu", wl.weights, wl.vectors, calls,
                    "the 4-bit decode layer with gate and up as one gated pair")


def draw_signs(rng, n: int) -> np.ndarray:
    return rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=n)


def f16_outproj_fwht_residual_4096(seed: int = 0) -> Workload:
    """The f16 4096x4096 residual projection reading the signed Hadamard
    transform of x (blocks of 1024, one random sign per element)."""
    rng = np.random.default_rng(seed)
    W = draw_float_weights(rng, "f16", 4096, 4096, 1.0 / 4096)
    x, r = draw_vec(rng, 4096), draw_vec(rng, 4096)
    sg = draw_signs(rng, 4096)
    calls = [Call("f16_fwht_outproj_add_inplace", "W", "x", "add", r="r", inplace=True, fwht=("s", 1024))]
    return Workload("f16_outproj_fwht_residual_4096", {"W": W}, {"x": x, "r": r, "s": sg}, calls,
                    "dst = W FWHT_1024(x * s) + r in place; W 4096x4096 f16, s +-1")


def f16_outproj_residual_4096_ncols8(seed: int = 0) -> Workload:
    """The f16 4096x4096 residual projection over eight destination columns
    (small-batch decode): x [8, 4096], residual [8, 4096], dst = W x_b + r_b in
    place."""
    rng = np.random.default_rng(seed)
    W = draw_float_weights(rng, "f16", 4096, 4096, 1.0 / 4096)
    x, r = draw_vec(rng, 8 * 4096), draw_vec(rng, 8 * 4096)
    calls = [Call("f16_outproj_add_inplace_ncols8", "W", "x", "add", r="r", inplace=True, ncols=8)]
    return Workload("f16_outproj_residual_4096_ncols8", {"W": W}, {"x": x, "r": r}, calls,
                    "W 4096x4096 f16 ~N(0,1/4096); eight columns, dst = W x_b + r_b in place")


def q4b32_gate_14336x4096_ncols4(seed: int = 0) -> Workload:
    """The 4-bit 4096->14336 silu gate over four destination columns."""
    rng = np.random.default_rng(seed)
    W = draw_q4b32(rng, 14336, 4096, 0.001, 0.02)
    x = draw_vec(rng, 4 * 4096)
    calls = [Call("q4_gate_silu_ncols4", "W", "x", "silu", ncols=4)]
    return Workload("q4b32_gate_14336x4096_ncols4", {"W": W}, {"x": x}, calls,
                    "4-bit 14336x4096 silu over four columns")


def bf16_swiglu_14336x4096_ncols4(seed: int = 0) -> Workload:
    """The bf16 gate and up projections of a 4096-hidden, 14336-FFN layer as
    one gated pair over four destination columns (small-batch decode)."""
    rng = np.random.default_rng(seed)
    Wg = draw_float_weights(rng, "bf16", 14336, 4096, 1.0 / 4096)
    Wu = draw_float_weights(rng, "bf16", 14336, 4096, 1.0 / 4096)
    x = draw_vec(rng, 4 * 4096)
    calls = [Call("bf16_gate_up_glu_ncols4", "Wgate", "x", "silu", w2="Wup", ncols=4)]
    return Workload("bf16_swiglu_14336x4096_ncols4", {"Wgate": Wg, "Wup": Wu}, {"x": x}, calls,
                    "bf16 14336x4096 gate and up, silu(W_g x_b) * (W_u x_b) over four columns")


WORKLOADS = {
    "f32_tiny_256": f32_tiny_256,
    "f16_outproj_residual_4096": f16_outproj_residual_4096,
    "bf16_swiglu_gate_14336x4096": bf16_swiglu_gate_14336x4096,
    "q8b32_view_residual_4096x6144": q8b32_view_residual_4096x6144,
    "q4b32_decode_layer": q4b32_decode_layer,
    "q4b32_decode_layer_glu": q4b32_decode_layer_glu,
    "f16_outproj_residual_4096_ncols8": f16_outproj_residual_4096_ncols8,
    "f16_outproj_fwht_residual_4096": f16_outproj_fwht_residual_4096,
    "q4b32_gate_14336x4096_ncols4": q4b32_gate_14336x4096_ncols4,
    "bf16_swiglu_14336x4096_ncols4": bf16_swiglu_14336x4096_ncols4,
}


def random_weights(rng, fmt: str, N: int, K: int) -> Weights:
    """Weights of any format and shape with the workloads' laws, for tests of
    odd shapes (float formats: variance 1/K; blocks: the 4-bit/8-bit laws)."""
    if fmt in ("f32", "f16", "bf16"):
        return draw_float_weights(rng, fmt, N, K, 1.0 / max(K, 1))
    if fmt == "q8b32":
        return draw_q8b32(rng, N, K, 0.001, 0.01)
    if fmt == "q4b32":
        return draw_q4b32(rng, N, K, 0.001, 0.02)
    raise ValueError(fmt)
