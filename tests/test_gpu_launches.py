"""Launches per 4-bit decode layer, counted by the HIP runtime.  The layer's
calls are captured from a stream into a graph (hipStreamBeginCapture /
hipStreamEndCapture), and the graph's kernel nodes are counted:
- fused: one launch per GEMV, 6;
- unfused: each GEMV without its epilogue plus a separate element-wise pass
  for each of the five that have one, 11;
- with gate and up as one gated pair: 5 fused, 10 unfused.
Unfused, the pair becomes up, gate and one silu(gate)*up pass."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from decode_gemv_elementwise_amd import binding, synth
from gpu_util import dev, log

pytestmark = pytest.mark.gpu

_KERNEL_NODE = 0       # hipGraphNodeTypeKernel
_CAPTURE_RELAXED = 2   # hipStreamCaptureModeRelaxed


def _hip():
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipStreamBeginCapture.argtypes = [ctypes.c_void_p, ctypes.c_int]
    hip.hipStreamEndCapture.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
    hip.hipGraphGetNodes.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_size_t)]
    hip.hipGraphNodeGetType.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int)]
    hip.hipGraphDestroy.argtypes = [ctypes.c_void_p]
    return hip


def _kernel_nodes(enqueue):
    """Kernel nodes in the graph captured from enqueue(stream_handle)."""
    hip = _hip()
    s = torch.cuda.Stream()
    h = s.cuda_stream
    enqueue(h)  # eager first: one-time function attributes are set outside capture
    torch.cuda.synchronize()
    assert hip.hipStreamBeginCapture(h, _CAPTURE_RELAXED) == 0
    enqueue(h)
    graph = ctypes.c_void_p()
    assert hip.hipStreamEndCapture(h, ctypes.byref(graph)) == 0
    n = ctypes.c_size_t(0)
    assert hip.hipGraphGetNodes(graph, None, ctypes.byref(n)) == 0
    nodes = (ctypes.c_void_p * n.value)()
    assert hip.hipGraphGetNodes(graph, nodes, ctypes.byref(n)) == 0
    kinds = []
    for i in range(n.value):
        t = ctypes.c_int(-1)
        assert hip.hipGraphNodeGetType(nodes[i], ctypes.byref(t)) == 0
        kinds.append(t.value)
    assert hip.hipGraphDestroy(graph) == 0
    return sum(1 for k in kinds if k == _KERNEL_NODE), len(kinds)


def _layer():
    wl = synth.q4b32_decode_layer(0)
    W = {n: (dev(w.data), w) for n, w in wl.weights.items()}
    v = {n: dev(a) for n, a in wl.vectors.items()}
    out = {n: torch.empty(w.N, dtype=torch.float32, device="cuda") for n, (_, w) in W.items()}
    tmp = {n: torch.empty(w.N, dtype=torch.float32, device="cuda") for n, (_, w) in W.items()}
    return W, v, out, tmp


def _gemv(W, name, x, act, dst, s, m=None, r=None):
    Wd, w = W[name]
    binding.gemv_fused(Wd, "q4b32", w.N, w.K, x, act, mul_operand=m, add_operand=r, dst=dst, stream=s)


def _epi(W, name, act, acc, dst, s, m=None, r=None):
    binding.gemv_epilogue(act, W[name][1].N, acc, mul_operand=m, add_operand=r, dst=dst, stream=s)


def test_launches_per_layer_fused_and_unfused():
    log("launch counts of the 4-bit layer")
    W, v, out, tmp = _layer()

    def fused(s):
        _gemv(W, "Wqkv", v["x_qkv"], "none", out["Wqkv"], s)
        _gemv(W, "Wo", v["x_o"], "add", out["Wo"], s, r=v["r_o"])
        _gemv(W, "Wgate", v["x_ffn"], "silu", out["Wgate"], s)
        _gemv(W, "Wup", v["x_ffn"], "mul", out["Wup"], s, m=out["Wgate"])
        _gemv(W, "Wdown", out["Wup"], "add", out["Wdown"], s, r=v["r_down"])
        _gemv(W, "Wg", v["x_g"], "sigmoid", out["Wg"], s)

    def unfused(s):
        _gemv(W, "Wqkv", v["x_qkv"], "none", out["Wqkv"], s)
        _gemv(W, "Wo", v["x_o"], "none", tmp["Wo"], s)
        _epi(W, "Wo", "add", tmp["Wo"], out["Wo"], s, r=v["r_o"])
        _gemv(W, "Wgate", v["x_ffn"], "none", tmp["Wgate"], s)
        _epi(W, "Wgate", "silu", tmp["Wgate"], out["Wgate"], s)
        _gemv(W, "Wup", v["x_ffn"], "none", tmp["Wup"], s)
        _epi(W, "Wup", "mul", tmp["Wup"], out["Wup"], s, m=out["Wgate"])
        _gemv(W, "Wdown", out["Wup"], "none", tmp["Wdown"], s)
        _epi(W, "Wdown", "add", tmp["Wdown"], out["Wdown"], s, r=v["r_down"])
        _gemv(W, "Wg", v["x_g"], "none", tmp["Wg"], s)
        _epi(W, "Wg", "sigmoid", tmp["Wg"], out["Wg"], s)

    kf, nf = _kernel_nodes(fused)
    ku, nu = _kernel_nodes(unfused)
    log(f"fused: {kf} kernel nodes of {nf}; unfused: {ku} of {nu}")
    assert (kf, ku) == (6, 11)
    assert nf == kf and nu == ku  # nothing but kernels: no memset or copy nodes


def test_launches_per_layer_with_gated_pair():
    log("launch counts of the 4-bit layer, gate and up as one gated pair")
    W, v, out, tmp = _layer()
    Wg_, wg = W["Wgate"]
    Wu_, _ = W["Wup"]

    def fused(s):
        _gemv(W, "Wqkv", v["x_qkv"], "none", out["Wqkv"], s)
        _gemv(W, "Wo", v["x_o"], "add", out["Wo"], s, r=v["r_o"])
        binding.gemv_glu(Wg_, Wu_, "q4b32", wg.N, wg.K, v["x_ffn"], "silu", dst=out["Wup"], stream=s)
        _gemv(W, "Wdown", out["Wup"], "add", out["Wdown"], s, r=v["r_down"])
        _gemv(W, "Wg", v["x_g"], "sigmoid", out["Wg"], s)

    def unfused(s):
        _gemv(W, "Wqkv", v["x_qkv"], "none", out["Wqkv"], s)
        _gemv(W, "Wo", v["x_o"], "none", tmp["Wo"], s)
        _epi(W, "Wo", "add", tmp["Wo"], out["Wo"], s, r=v["r_o"])
        _gemv(W, "Wup", v["x_ffn"], "none", tmp["Wup"], s)
        _gemv(W, "Wgate", v["x_ffn"], "none", tmp["Wgate"], s)
        _epi(W, "Wgate", "silu_mul", tmp["Wgate"], out["Wup"], s, m=tmp["Wup"])
        _gemv(W, "Wdown", out["Wup"], "none", tmp["Wdown"], s)
        _epi(W, "Wdown", "add", tmp["Wdown"], out["Wdown"], s, r=v["r_down"])
        _gemv(W, "Wg", v["x_g"], "none", tmp["Wg"], s)
        _epi(W, "Wg", "sigmoid", tmp["Wg"], out["Wg"], s)

    kf, nf = _kernel_nodes(fused)
    ku, nu = _kernel_nodes(unfused)
    log(f"gated pair fused: {kf} kernel nodes of {nf}; unfused: {ku} of {nu}")
    assert (kf, ku) == (5, 10)
    assert nf == kf and nu == ku
