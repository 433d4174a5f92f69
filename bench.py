#!/usr/bin/env python3
"""Benchmark of the fused-epilogue decode GEMV on one MI355X.

A step is one pass of the whole path over one synthetic input: for the
default workload (one 4-bit decode layer), the six gemv_fused calls of the
layer, each staging x in LDS, streaming its W from HBM, dequantising in
registers, reducing each row over its wave and applying its epilogue before
the one store.  Inputs are resident in HBM before timing starts.  W (and x,
the operands and dst) rotate over enough copies to exceed 512 MiB, so the
256 MB Infinity Cache cannot serve W from a previous step.

The timed steps are captured once into a HIP graph (the calls' host checks
run at capture) and the graph is replayed between two HIP events recorded on
the launch stream; the replay of exactly `steps` steps is timed `repeats`
times and the line reports the median (and the minimum).  `--launch stream`
launches every call from the host instead, host checks included.

value = algorithmic bytes per step x steps / time, in GB/s, where algorithmic
bytes = W in its storage format + 4K (x) + 4N per epilogue operand read + 4N
(dst).  One JSON line per workload on stdout.
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "fused GEMV achieved HBM GB/s (% of peak) and µs/call at decode shapes"
PEAK_HBM_GBPS = 8000.0
# f32 FMA throughput of the vector ALUs without packed FP32 (the kernels are
# built with packed FP32 off): 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz
PEAK_VALU_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
# dense f16 matrix-core peak (the matrix-core column kernel runs f16 MFMAs)
PEAK_MFMA_F16_TFLOPS = 2500.0
ROTATE_MIN_BYTES = 512 << 20
DEFAULT_WORKLOAD = "q4b32_decode_layer"
# the library's device code (every kernel a counter or trace summary can
# cover; host checks excluded): a summary stays valid while these files are
# unchanged
KERNEL_SOURCES = [os.path.join(ROOT, "decode_gemv_elementwise_amd", "csrc", f)
                  for f in ("gemv_device.h", "gemv_fast.h", "gemv_kernels.hip", "gemv_cols.hip",
                            "gemv_mfma.hip", "gemv_fwht.hip")]
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--repeats", type=int, default=10, help="timed replays of the `steps` steps (median and minimum reported)")
    p.add_argument("--workload", default=DEFAULT_WORKLOAD,
                   help="a workload name, or 'all' (one JSON line each)")
    p.add_argument("--launch", choices=["graph", "stream"], default="graph")
    p.add_argument("--unfused", action="store_true",
                   help="time gemv_fused(none) + gemv_epilogue as the primary figure instead of the fused call")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="CPU-oracle sample length (0 disables the CPU legs)")
    p.add_argument("--no-probe", action="store_true", help="skip the bandwidth probe and the floor measurements")
    p.add_argument("--skip-other", action="store_true",
                   help="do not also time the opposite composition (fused vs unfused), so that a profiler's "
                        "trace holds only the primary one's kernels")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="only run a plain device copy of BYTES bytes, 5 times (calibrates the "
                        "FETCH_SIZE / WRITE_SIZE counters against a known byte count), then exit")
    return p.parse_args()


def probe_lib():
    import ctypes
    from decode_gemv_elementwise_amd import build as b
    lib = ctypes.CDLL(b.PROBE_LIB)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.hbm_read_probe.argtypes = [vp, i64, vp, ctypes.c_int, vp]
    lib.hbm_copy.argtypes = [vp, vp, i64, vp]
    lib.hbm_read_floor.argtypes = [vp, i64, vp, ctypes.c_int, vp]
    lib.hbm_read_floor_out_floats.argtypes = [i64, ctypes.c_int]
    lib.hbm_read_floor_out_floats.restype = i64
    lib.hbm_read_floor_shapes.restype = ctypes.c_int
    lib.gemv_valu_floor.argtypes = [ctypes.c_int, i64, i64, vp, vp, vp]
    lib.hbm_read_once.argtypes = [vp, i64, vp, vp]
    lib.hbm_read_once_blocks.argtypes = [i64]
    return lib


def copy_calibration(torch, nbytes):
    lib = probe_lib()
    nbytes = (nbytes + 15) // 16 * 16
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.zeros_like(src)
    s = torch.cuda.current_stream().cuda_stream
    for _ in range(5):
        rc = lib.hbm_copy(src.data_ptr(), dst.data_ptr(), nbytes, s)
        if rc != 0:
            sys.exit(f"hbm_copy failed: {rc}")
    torch.cuda.synchronize()
    assert bool(torch.equal(src, dst))
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 5}), flush=True)


# ------------------------------------------------------------------ setup

def kernel_sha():
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        h.update(open(path, "rb").read())
    return h.hexdigest()


def align(v, a=256):
    return (v + a - 1) // a * a


def call_bytes(wl, c):
    w = wl.weights[c.w]
    ops = (1 if c.m else 0) + (1 if c.r else 0)
    w2 = wl.weights[c.w2].data.size if c.w2 else 0
    signs = 4 * wl.vectors[c.fwht[0]].size if c.fwht else 0
    return w.data.size + w2 + signs + c.ncols * (4 * w.K + 4 * w.N * ops + 4 * w.N)


class Step:
    """Device copies of one workload, R rotating sets, and the prepared calls
    of every set (fused, or the unfused composition)."""

    def __init__(self, torch, binding, wl, unfused: bool):
        self.wl = wl
        self.calls = wl.calls
        per_set = sum(w.data.size for w in wl.weights.values())
        self.copies = max(2, -(-ROTATE_MIN_BYTES // per_set))
        R = self.copies
        dev = "cuda"
        # one allocation per tensor kind, each set at a 256-byte aligned offset
        self.w_slot = {k: align(w.data.size) for k, w in wl.weights.items()}
        self.w_buf = {}
        for k, w in wl.weights.items():
            buf = torch.empty(R * self.w_slot[k], dtype=torch.uint8, device=dev)
            src = torch.from_numpy(w.data).to(dev)
            for i in range(R):
                buf[i * self.w_slot[k]: i * self.w_slot[k] + w.data.size].copy_(src)
            self.w_buf[k] = buf
        self.v_buf = {}
        for k, v in wl.vectors.items():
            t = torch.from_numpy(np.ascontiguousarray(v).reshape(-1)).to(dev)
            self.v_buf[k] = torch.stack([t.clone() for _ in range(R)])
        self.out_buf = {c.name: torch.zeros((R, c.ncols * wl.weights[c.w].N), dtype=torch.float32, device=dev)
                        for c in self.calls}
        self.tmp_buf = {c.name: torch.zeros((R, c.ncols * wl.weights[c.w].N), dtype=torch.float32, device=dev)
                        for c in self.calls}
        self.up_buf = {c.name: torch.zeros((R, c.ncols * wl.weights[c.w].N), dtype=torch.float32, device=dev)
                       for c in self.calls if c.w2}
        self.xt_buf = {c.name: torch.zeros((R, wl.weights[c.w].K), dtype=torch.float32, device=dev)
                       for c in self.calls if c.fwht}
        self.prepared = []
        for i in range(R):
            self.prepared.append(self._prepare_set(binding, i, unfused))
        self.bytes_per_step = sum(call_bytes(wl, c) for c in self.calls)

    def _vec(self, name, i, shape=None):
        if name is None:
            return None
        if name.startswith("@"):
            t = self.out_buf[name[1:]][i]
        else:
            t = self.v_buf[name][i]
        return t.view(shape) if shape else t

    def _prepare_set(self, binding, i, unfused):
        fns = []
        for c in self.calls:
            w = self.wl.weights[c.w]
            W = self.w_buf[c.w][i * self.w_slot[c.w]:]
            x = self._vec(c.x, i)
            shape = c.out_shape or ((w.N,) if c.ncols == 1 else (c.ncols, w.N))
            m = self._vec(c.m, i, shape)
            r = self._vec(c.r, i, shape)
            if c.inplace:
                dst = r if c.act == "add" else m
            else:
                dst = self.out_buf[c.name][i].view(shape)
            if c.w2 and c.ncols > 1:
                W2 = self.w_buf[c.w2][i * self.w_slot[c.w2]:]
                if unfused:  # up (none), gate (none) over the columns, then silu(gate) * up
                    up, tmp = self.up_buf[c.name][i].view(shape), self.tmp_buf[c.name][i].view(shape)
                    fns.append(binding.PreparedNcols(W2, w.fmt, w.N, w.K, c.ncols, x, "none", dst=up))
                    fns.append(binding.PreparedNcols(W, w.fmt, w.N, w.K, c.ncols, x, "none", dst=tmp))
                    fns.append(_PreparedEpilogue(binding, "silu_mul", c.ncols * w.N, tmp, up, None, dst))
                else:
                    fns.append(binding.PreparedGluNcols(W, W2, w.fmt, w.N, w.K, c.ncols, x, c.act, dst=dst))
            elif c.w2:
                W2 = self.w_buf[c.w2][i * self.w_slot[c.w2]:]
                if unfused:  # up (none), gate (none), then silu(gate) * up
                    up, tmp = self.up_buf[c.name][i], self.tmp_buf[c.name][i]
                    fns.append(binding.PreparedCall(W2, w.fmt, w.N, w.K, x, "none", dst=up))
                    fns.append(binding.PreparedCall(W, w.fmt, w.N, w.K, x, "none", dst=tmp))
                    fns.append(_PreparedEpilogue(binding, "silu_mul", w.N, tmp, up, None, dst))
                else:
                    fns.append(binding.PreparedGlu(W, W2, w.fmt, w.N, w.K, x, c.act, dst=dst))
            elif c.fwht:
                sg = self._vec(c.fwht[0], i)
                n = c.fwht[1]
                if unfused:  # the transform into a buffer, then the product reading it
                    xt = self.xt_buf[c.name][i]
                    fns.append(binding.PreparedFwht(x, sg, 1, w.K, n, sg.numel(), xt))
                    fns.append(binding.PreparedCall(W, w.fmt, w.N, w.K, xt, c.act, mul_operand=m, add_operand=r,
                                                    dst=dst))
                else:
                    fns.append(binding.PreparedFusedFwht(W, w.fmt, w.N, w.K, x, sg, n, sg.numel(), c.act,
                                                         mul_operand=m, add_operand=r, dst=dst))
            elif c.ncols > 1:
                if unfused and c.act != "none":
                    tmp = self.tmp_buf[c.name][i].view(shape)
                    fns.append(binding.PreparedNcols(W, w.fmt, w.N, w.K, c.ncols, x, "none", dst=tmp))
                    fns.append(_PreparedEpilogue(binding, c.act, c.ncols * w.N, tmp, m, r, dst))
                else:
                    fns.append(binding.PreparedNcols(W, w.fmt, w.N, w.K, c.ncols, x, c.act, mul_operand=m,
                                                     add_operand=r, dst=dst))
            elif unfused and c.act != "none":
                tmp = self.tmp_buf[c.name][i]
                fns.append(binding.PreparedCall(W, w.fmt, w.N, w.K, x, "none", dst=tmp))
                fns.append(_PreparedEpilogue(binding, c.act, w.N, tmp, m, r, dst))
            else:
                fns.append(binding.PreparedCall(W, w.fmt, w.N, w.K, x, c.act, mul_operand=m, add_operand=r,
                                                dst=dst))
        return fns

    def launches_per_step(self):
        return len(self.prepared[0])


class _PreparedEpilogue:
    def __init__(self, binding, act, N, acc, m, r, dst):
        self.args = (act, N, acc, m, r, dst)
        self.binding = binding

    def __call__(self):
        act, N, acc, m, r, dst = self.args
        self.binding.gemv_epilogue(act, N, acc, mul_operand=m, add_operand=r, dst=dst)


def run_steps(step, n, offset=0):
    R = step.copies
    for s in range(n):
        for fn in step.prepared[(offset + s) % R]:
            fn()


def time_steps(torch, step, steps, warmup, launch, repeats):
    """Seconds for exactly `steps` steps, once per repeat, after `warmup`
    untimed ones; each timed region is bracketed by device synchronisations
    and measured with HIP events on the stream the kernels are launched on."""
    stream = torch.cuda.Stream()
    out = []
    with torch.cuda.stream(stream):
        run_steps(step, 1)  # first launch outside any capture
        torch.cuda.synchronize()
        if launch == "graph":
            gw = torch.cuda.CUDAGraph() if warmup > 0 else None
            if gw is not None:
                with torch.cuda.graph(gw, stream=stream):
                    run_steps(step, warmup)
            gt = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gt, stream=stream):
                run_steps(step, steps, offset=warmup)
            torch.cuda.synchronize()
            if gw is not None:
                gw.replay()
            for _ in range(repeats):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record(stream)
                gt.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                out.append(e0.elapsed_time(e1) / 1e3)
            del gt, gw
        else:
            run_steps(step, warmup)
            for _ in range(repeats):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record(stream)
                run_steps(step, steps, offset=warmup)
                e1.record(stream)
                torch.cuda.synchronize()
                out.append(e0.elapsed_time(e1) / 1e3)
    return out


def probe_bandwidth(torch, nbytes=2 << 30):
    lib = probe_lib()
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    blocks = 2048
    out = torch.zeros(blocks, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        assert lib.hbm_read_probe(buf.data_ptr(), nbytes, out.data_ptr(), blocks, s) == 0
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    reps = 10
    for _ in range(reps):
        lib.hbm_read_probe(buf.data_ptr(), nbytes, out.data_ptr(), blocks, s)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    ok = float(out.sum()) == nbytes / 4
    del buf
    return nbytes / sec / 1e9, ok


def replay_us(torch, launch_one, n, repeats=3):
    """Median per-launch microseconds of n launches captured in one graph on a
    stream of its own, replayed `repeats` times; launch_one(i, stream) issues
    launch i."""
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        launch_one(0, stream.cuda_stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                launch_one(i, stream.cuda_stream)
        g.replay()
        torch.cuda.synchronize()
        t = []
        for _ in range(repeats):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) * 1e3 / n)
    del g
    return float(np.median(t))


def read_floor_us(torch, nbytes, n):
    """Per-launch time of reading nbytes and storing one result per wave, in
    each of the probe library's launch shapes, over rotating buffers totalling
    more than 512 MiB, replayed as a graph like the GEMV: {shape: us}."""
    lib = probe_lib()
    nbytes = (nbytes + 15) // 16 * 16
    slot = (nbytes + 4095) // 4096 * 4096
    copies = max(2, -(-(512 << 20) // slot))
    buf = torch.ones(copies * slot // 4, dtype=torch.float32, device="cuda")
    res = {}
    names = {0: "one pass, 4-wave workgroups, 8 loads per lane",
             1: "one pass, 16-wave workgroups, 4 loads per lane",
             2: "resident grid, 16-wave workgroups, 4 loads per lane per step"}
    for shape in range(lib.hbm_read_floor_shapes()):
        # the results rotate with the inputs, as a GEMV's dst does (a launch
        # that stores over the previous launch's lines pays for it)
        nout = int(lib.hbm_read_floor_out_floats(nbytes, shape))
        oslot = (nout + 63) // 64 * 64
        out = torch.zeros(copies * oslot, dtype=torch.float32, device="cuda")

        def one(i, s, shape=shape, out=out, oslot=oslot):
            rc = lib.hbm_read_floor(buf.data_ptr() + (i % copies) * slot, nbytes,
                                    out.data_ptr() + 4 * (i % copies) * oslot, shape, s)
            assert rc == 0, rc
        res[names.get(shape, str(shape))] = round(replay_us(torch, one, n), 3)
        del out
    del buf
    torch.cuda.empty_cache()
    return res


def read_only_us(torch, nbytes, n):
    """Per-launch time of merely reading nbytes in one pass (4-wave
    workgroups, 8 loads per lane), with no store a launch must wait for, over
    the same rotating buffers and graph replay: what the store of the read +
    store floor adds is the difference."""
    lib = probe_lib()
    nbytes = (nbytes + 15) // 16 * 16
    slot = (nbytes + 4095) // 4096 * 4096
    copies = max(2, -(-(512 << 20) // slot))
    buf = torch.ones(copies * slot // 4, dtype=torch.float32, device="cuda")
    nout = int(lib.hbm_read_once_blocks(nbytes))
    oslot = (nout + 63) // 64 * 64
    out = torch.zeros(copies * oslot, dtype=torch.float32, device="cuda")

    def one(i, s):
        assert lib.hbm_read_once(buf.data_ptr() + (i % copies) * slot, nbytes,
                                 out.data_ptr() + 4 * (i % copies) * oslot, s) == 0
    us = round(replay_us(torch, one, n), 3)
    del buf, out
    torch.cuda.empty_cache()
    return us


def valu_floor_us(torch, fmt, N, K, n):
    """Per-launch time of the one-column kernel's arithmetic alone for an
    N x K call (the probe library's gemv_valu_floor): no weight byte read."""
    from decode_gemv_elementwise_amd import binding
    lib = probe_lib()
    x = torch.ones(64, dtype=torch.float32, device="cuda")
    out = torch.zeros(N, dtype=torch.float32, device="cuda")

    def one(i, s):
        assert lib.gemv_valu_floor(binding.FORMATS[fmt], N, K, x.data_ptr(), out.data_ptr(), s) == 0
    return round(replay_us(torch, one, n), 3)


def stream_us_per_call(torch, fns, n=400):
    """Host-inclusive microseconds per call: prepared calls (one per rotating
    set, taken in turn) launched n times back to back from Python on one
    stream, timed on the host: the library's argument checks, the launch, the
    Python/ctypes marshalling and the kernel itself."""
    for i in range(20):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / n * 1e6


# ------------------------------------------------------------------ CPU legs

def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def host_threads():
    """The threads this process may use: its CPU affinity, capped by
    OMP_NUM_THREADS where that is set (the GPU machine's share of the host)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def _oracle_call(oracle, wl, c, outputs, rows=None):
    w = wl.weights[c.w]
    x = outputs[c.x[1:]] if c.x.startswith("@") else wl.vectors[c.x]
    m = (outputs[c.m[1:]] if c.m.startswith("@") else wl.vectors[c.m]) if c.m else None
    r = wl.vectors[c.r] if c.r else None
    if c.w2 and c.ncols > 1:
        return oracle.glu_ncols_reference(w.fmt, w.N, w.K, w.data, wl.weights[c.w2].data,
                                          np.reshape(x, (c.ncols, w.K)), c.act, rows=rows)[0]
    if c.w2:
        return oracle.glu_reference(w.fmt, w.N, w.K, w.data, wl.weights[c.w2].data, x, c.act, rows=rows)[0]
    if c.fwht:
        return oracle.fwht_gemv_reference(w.fmt, w.N, w.K, w.data, x, wl.vectors[c.fwht[0]], c.fwht[1], c.act,
                                          m=m, r=r, rows=rows)[0]
    if c.ncols > 1:
        M = None if m is None else np.reshape(m, (c.ncols, w.N))
        R = None if r is None else np.reshape(r, (c.ncols, w.N))
        return oracle.ncols_reference(w.fmt, w.N, w.K, w.data, np.reshape(x, (c.ncols, w.K)), c.act,
                                      M=M, R=R, rows=rows)[0]
    return oracle.reference(w.fmt, w.N, w.K, w.data, x, c.act, m=m, r=r, rows=rows)[0]


def _oracle_step(oracle, wl, threads, pool):
    """One pass of the workload through the oracle; with threads > 1 each call's
    rows are split into contiguous ranges run concurrently (the C oracle runs
    without the interpreter lock), so every row is computed by the same code
    in the same order as with one thread."""
    outputs = {}
    for c in wl.calls:
        N = wl.weights[c.w].N
        if threads == 1:
            y = _oracle_call(oracle, wl, c, outputs)
        else:
            bounds = [(N * k // threads, N * (k + 1) // threads) for k in range(threads)]
            parts = list(pool.map(lambda b: _oracle_call(oracle, wl, c, outputs, rows=b),
                                  [b for b in bounds if b[1] > b[0]]))
            y = np.concatenate(parts, axis=-1)
        outputs[c.name] = np.asarray(y).astype(np.float32).reshape(-1)
    return outputs


def cpu_baseline(wl, seconds):
    """The oracle as written (double precision, every row, each epilogue as its
    own pass) on the GPU machine's host over full steps of the same workload: on
    one thread for about `seconds`, then row-partitioned over every host
    thread for about half that; both runs give bit-identical outputs."""
    import oracle
    step_bytes = sum(call_bytes(wl, c) for c in wl.calls)
    res = {}
    ref = None
    threads_all = host_threads()
    for threads, budget in ((1, seconds), (threads_all, seconds / 2)):
        with ThreadPoolExecutor(max_workers=threads) as pool:
            t0 = time.perf_counter()
            steps = 0
            while True:
                out = _oracle_step(oracle, wl, threads, pool)
                steps += 1
                el = time.perf_counter() - t0
                if el >= budget:
                    break
        if ref is None:
            ref = out
        same = all(np.array_equal(ref[k].view(np.uint32), out[k].view(np.uint32)) for k in ref)
        res[threads] = (steps, el, same)
    steps1, el1, _ = res[1]
    stepsn, eln, same = res[threads_all]
    return {"value": round(step_bytes * steps1 / el1 / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps1} full steps of {wl.name} ({len(wl.calls)} calls each: every row, double "
                      f"accumulation, separate epilogue pass) in {el1:.1f} s on one host thread",
            "us_per_step": round(el1 / steps1 * 1e6, 1),
            "cpu_model": cpu_model(), "nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
            "all_cores": {"value": round(step_bytes * stepsn / eln / 1e9, 4), "unit": "GB/s",
                          "threads": threads_all, "us_per_step": round(eln / stepsn * 1e6, 1),
                          "sample": f"{stepsn} full steps in {eln:.1f} s, each call's rows split over "
                                    f"{threads_all} threads", "bitwise_equal_to_one_thread": bool(same)}}


def cpu_fused_baseline(wl, seconds):
    """The CPU comparison GEMV (tile-fused epilogue, AVX2 vectors, every host
    core) on the same workload's full calls, fused and unfused, for about
    `seconds` of wall time each; None when a call kind has no CPU path."""
    from decode_gemv_elementwise_amd import cpu_fused
    if not cpu_fused.available():
        return None
    if any(c.w2 or c.ncols > 1 or c.fwht for c in wl.calls):
        return None
    threads = host_threads()
    out = {}
    for fused in (True, False):
        outputs = {}
        t0 = time.perf_counter()
        steps = 0
        while True:
            for c in wl.calls:
                w = wl.weights[c.w]
                x = outputs[c.x[1:]] if c.x.startswith("@") else wl.vectors[c.x]
                m = (outputs[c.m[1:]] if c.m.startswith("@") else wl.vectors[c.m]) if c.m else None
                r = wl.vectors[c.r] if c.r else None
                outputs[c.name] = cpu_fused.gemv(w.fmt, w.N, w.K, w.data, x, c.act, m=m, r=r, threads=threads,
                                                 fused=fused)
            steps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        out["fused" if fused else "unfused"] = el / steps
    nbytes = sum(wl.weights[c.w].data.size + 4 * wl.weights[c.w].K
                 + 4 * wl.weights[c.w].N * (1 + (1 if c.m else 0) + (1 if c.r else 0)) for c in wl.calls)
    return {"value": round(nbytes / out["fused"] / 1e9, 3), "unit": "GB/s", "threads": threads,
            "kind": "tile-fused vectorised CPU GEMV", "us_per_step": round(out["fused"] * 1e6, 1),
            "unfused_us_per_step": round(out["unfused"] * 1e6, 1),
            "sample": f"full steps of {wl.name} for about {seconds:.0f} s each, fused and unfused, "
                      f"{threads} host threads"}


# ------------------------------------------------------------------ committed profiles

def _read_summary(path):
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_sha():
        return None
    return kv


def read_counters(workload):
    """Per-launch HBM traffic (bytes) of this workload's dominant kernel from
    the committed rocprofv3 counter summary, if it was taken on the current
    kernel source; else None."""
    kv = _read_summary(os.path.join(PROFILES, f"counters_{workload}.txt"))
    try:
        return None if kv is None else float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_trace(workload):
    """Average device durations (us) of this workload's dominant kernel and of
    the best read + store floor kernel traced beside it, from the committed
    rocprofv3 kernel-trace summary, if it was taken on the current kernel
    source; else None for each."""
    kv = _read_summary(os.path.join(PROFILES, f"trace_{workload}.txt"))

    def us(key):
        try:
            return float(kv[key].split()[0]) / 1e3
        except (KeyError, ValueError, IndexError, TypeError):
            return None
    return us("dominant_kernel_avg_ns"), us("trace_read_store_floor_avg_ns")


# ------------------------------------------------------------------ one workload

def _alone(synth, wl, dom):
    """The dominant call as a workload of its own; inputs that earlier calls
    of the step produce become fresh vectors of the same length (timing only)."""
    vecs = dict(wl.vectors)
    w = wl.weights[dom.w]
    x, m = dom.x, dom.m
    if x.startswith("@"):
        x = "_x_alone"
        vecs[x] = synth.draw_vec(np.random.default_rng(1), dom.ncols * w.K)
    if m and m.startswith("@"):
        m = "_m_alone"
        vecs[m] = synth.draw_vec(np.random.default_rng(2), dom.ncols * w.N)
    alone = synth.Call(dom.name, dom.w, x, dom.act, m=m, r=dom.r, out_shape=dom.out_shape,
                       inplace=dom.inplace, w2=dom.w2, ncols=dom.ncols, fwht=dom.fwht)
    ws = {dom.w: w}
    if dom.w2:
        ws[dom.w2] = wl.weights[dom.w2]
    return synth.Workload(wl.name, ws, vecs, [alone])


def _kernel_name(binding, dom, w, cols_kernel):
    if dom.w2 and dom.ncols > 1:
        return (f"gemv_cols_mfma_kernel<{w.fmt}, ncols={dom.ncols}> x2, gated pair as up then gate ({dom.name})"
                if cols_kernel == "columns_matrix" and dom.act == "silu" else
                f"gemv_cols(_tiles)_kernel<{w.fmt}, ncols={dom.ncols}, gated pair> ({dom.name})")
    if cols_kernel == "columns_matrix":
        return f"gemv_cols_mfma_kernel<{w.fmt}, ncols={dom.ncols}> ({dom.name})"
    if dom.ncols > 1:
        return f"gemv_cols_kernel<{w.fmt}, ncols={dom.ncols}> ({dom.name})"
    if dom.fwht:
        return f"gemv_fast_kernel<{w.fmt}, signed Hadamard prologue> ({dom.name})"
    return f"gemv_fast_kernel<{w.fmt}{', gated pair' if dom.w2 else ''}> ({dom.name})"


def bench_workload(torch, binding, synth, name, args, probe):
    wl = synth.WORKLOADS[name](0)
    log(f"workload {name}: preparing rotating copies")
    step = Step(torch, binding, wl, args.unfused)
    log(f"  {step.copies} copies, {step.launches_per_step()} launches/step, "
        f"{step.bytes_per_step} algorithmic bytes/step")
    secs = time_steps(torch, step, args.steps, args.warmup, args.launch, args.repeats)
    sec = float(np.median(secs))
    ms_per_step = sec / args.steps * 1e3
    value = step.bytes_per_step * args.steps / sec / 1e9
    log(f"  {ms_per_step * 1e3:.3f} us/step (median of {len(secs)}), min {min(secs) / args.steps * 1e6:.3f}")

    # the same step with every epilogue as a separate pass (the fusion effect)
    other = None
    if not args.skip_other and any(c.act != "none" or c.w2 or c.fwht for c in wl.calls):
        ostep = Step(torch, binding, wl, not args.unfused)
        osecs = time_steps(torch, ostep, args.steps, args.warmup, args.launch, args.repeats)
        other = {"us_per_step": round(float(np.median(osecs)) / args.steps * 1e6, 3),
                 "launches_per_step": ostep.launches_per_step()}
        del ostep

    # dominant kernel: the call with the most bytes, timed alone the same way
    dom = max(wl.calls, key=lambda c: call_bytes(wl, c))
    if len(wl.calls) == 1 and step.launches_per_step() == 1:
        dom_secs = [s / args.steps for s in secs]
        dstep = step
    else:
        dstep = Step(torch, binding, _alone(synth, wl, dom), False)
        dom_secs = [s / args.steps for s in time_steps(torch, dstep, args.steps, args.warmup, args.launch,
                                                       args.repeats)]
    dom_sec = float(np.median(dom_secs))
    stream_us = (stream_us_per_call(torch, [p[0] for p in dstep.prepared]) if dstep.launches_per_step() == 1
                 else None)
    del dstep
    dom_bytes = call_bytes(wl, dom)
    dom_w = wl.weights[dom.w]
    dom_flops = 2 * dom_w.N * dom_w.K * dom.ncols * (2 if dom.w2 else 1)
    achieved = dom_bytes / dom_sec / 1e9
    cols_kernel = binding.gemv_ncols_kernel(dom_w.fmt, dom_w.N, dom_w.K, dom.ncols) if dom.ncols > 1 else None
    traffic = read_counters(name)
    trace_us, trace_floor_us = read_trace(name)
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": name, "calls": [
            {"name": c.name, "wfmt": wl.weights[c.w].fmt, "N": wl.weights[c.w].N, "K": wl.weights[c.w].K,
             "epilogue": (f"{c.act}(gate) * up" if c.w2 else c.act) + (" in place" if c.inplace else "")
             + (f" view {list(c.out_shape)}" if c.out_shape else ""), **({"ncols": c.ncols} if c.ncols > 1 else {}),
             **({"prologue": f"signed FWHT n={c.fwht[1]}"} if c.fwht else {})}
            for c in wl.calls],
            "fused": not args.unfused, "launches_per_step": step.launches_per_step(),
            "launch": args.launch, "rotating_copies": step.copies, "repeats": args.repeats,
            "algorithmic_bytes_per_step": step.bytes_per_step},
        "us_per_step": round(ms_per_step * 1e3, 3),
        "us_per_step_min": round(min(secs) / args.steps * 1e6, 3),
        "pct_of_hbm_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "kernel": _kernel_name(binding, dom, dom_w, cols_kernel),
                     "algorithmic_bytes_per_launch": dom_bytes,
                     "us_per_launch": round(dom_sec * 1e6, 3),
                     "us_per_launch_min": round(min(dom_secs) * 1e6, 3),
                     "trace_us_per_launch": None if trace_us is None else round(trace_us, 3),
                     "trace_same_size_read_store_us": None if trace_floor_us is None else round(trace_floor_us, 3),
                     "stream_us_per_call": None if stream_us is None else round(stream_us, 3)},
    }
    if other is not None:
        res["unfused" if not args.unfused else "fused_step"] = other
    # one FMA per weight and destination column: where that work at the peak
    # of the units that run it (the matrix cores for the matrix-core column
    # kernel, else the vector ALUs) takes longer than the bytes at the HBM
    # peak, the ALU is the roof
    peak_flops = PEAK_MFMA_F16_TFLOPS if cols_kernel == "columns_matrix" else PEAK_VALU_TFLOPS
    if dom_flops / (peak_flops * 1e12) > dom_bytes / (PEAK_HBM_GBPS * 1e9):
        tflops = dom_flops / dom_sec / 1e12
        res["roofline"].update({"bound": "alu" if peak_flops == PEAK_VALU_TFLOPS else "mfma",
                                "achieved": round(tflops, 3), "peak": round(peak_flops, 1),
                                "unit": "TFLOP/s", "frac": round(tflops / peak_flops, 4),
                                "algorithmic_flops_per_launch": dom_flops,
                                "hbm_gbps": round(achieved, 2)})
    if probe is not None:
        res["probe_read_gbps"] = round(probe, 1)
        res["roofline"]["frac_of_probe"] = round(achieved / probe, 4)
        # the same bytes read by kernels that do nothing else, each wave then
        # storing one result as a GEMV launch must: the best of three launch
        # shapes is what the launch and the stream alone cost at this size
        floors = read_floor_us(torch, dom_bytes, max(50, min(args.steps, 400)))
        floor_us = min(floors.values())
        res["roofline"]["same_size_read_store_us"] = floor_us
        res["roofline"]["same_size_read_store_by_shape_us"] = floors
        res["roofline"]["frac_of_same_size_read_store"] = round(floor_us / (dom_sec * 1e6), 4)
        res["roofline"]["frac_of_peak_at_floor"] = round(dom_bytes / (floor_us * 1e3) / PEAK_HBM_GBPS, 4)
        res["roofline"]["same_size_read_only_us"] = read_only_us(torch, dom_bytes, max(50, min(args.steps, 400)))
        if dom.ncols == 1 and not dom.w2 and not dom.fwht:
            # the kernel's arithmetic alone, no weight byte read
            res["roofline"]["valu_floor_us"] = valu_floor_us(torch, dom_w.fmt, dom_w.N, dom_w.K,
                                                             max(50, min(args.steps, 400)))
    del step
    torch.cuda.empty_cache()
    return res, wl


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the fused GEMV has no multi-GPU path in this "
              "library (row or K sharding is described in the design notes); use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.repeats < 1:
        sys.exit("steps and repeats must be >= 1 and warmup >= 0")
    import torch
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    if args.copy_calibration > 0:
        copy_calibration(torch, args.copy_calibration)
        return
    from decode_gemv_elementwise_amd import binding, synth
    binding.load()  # fails loudly if the HIP library is not built

    probe = None
    if not args.no_probe:
        probe, ok = probe_bandwidth(torch)
        log(f"read probe: {probe:.1f} GB/s (sum check {'ok' if ok else 'FAILED'})")
    names = list(synth.WORKLOADS) if args.workload == "all" else [args.workload]
    # the CPU legs run once: on the default workload, else on the first one
    cpu_on = DEFAULT_WORKLOAD if DEFAULT_WORKLOAD in names else names[0]
    for name in names:
        res, wl = bench_workload(torch, binding, synth, name, args, probe)
        if name == cpu_on and args.cpu_seconds > 0:
            log("cpu baseline (oracle, one thread, then every host thread)")
            res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
            log("cpu comparison (tile-fused GEMV, every host thread)")
            res["cpu_fused"] = cpu_fused_baseline(wl, args.cpu_seconds / 2)
        print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
