#!/usr/bin/env python3
"""Benchmark of the fused-epilogue decode GEMV on one MI355X.

A step is one pass of the whole path over one synthetic input: one
gemv_fused call (validate + launch, x staged into LDS, W streamed from HBM,
dequantised in registers, dot product, wave reduction, epilogue, store); for
the 4-bit layer workload, the six calls of the layer.  Inputs are resident in
HBM before timing starts.  W (and x, operands, dst) rotate over enough copies
to exceed 512 MiB, so the 256 MB Infinity Cache cannot serve W from a
previous step.  The timed steps are captured in one HIP graph and replayed
between two HIP events recorded on the launch stream.

value = algorithmic bytes per step x steps / time, in GB/s, where algorithmic
bytes = W in its storage format + 4K (x) + 4N per epilogue operand read + 4N
(dst).  One JSON line on stdout.
"""
import argparse
import hashlib
import json
import os
import sys
import time

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
DEFAULT_WORKLOAD = "f16_outproj_residual_4096"
# the device code of the one-column kernel (the kernel the counter summaries
# cover; entry points and host checks excluded): a summary stays valid while
# these files are unchanged
KERNEL_SOURCES = [os.path.join(ROOT, "decode_gemv_elementwise_amd", "csrc", f)
                  for f in ("gemv_device.h", "gemv_fast.h")]
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD,
                   help="a workload name, or 'all' (one JSON line each)")
    p.add_argument("--launch", choices=["graph", "stream"], default="graph")
    p.add_argument("--unfused", action="store_true",
                   help="time gemv_fused(none) + gemv_epilogue instead of the fused call")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="CPU-oracle sample length (0 disables the cpu_baseline leg)")
    p.add_argument("--no-probe", action="store_true", help="skip the read-bandwidth probe")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="only run a plain device copy of BYTES bytes, 5 times (calibrates the "
                        "FETCH_SIZE / WRITE_SIZE counters against a known byte count), then exit")
    return p.parse_args()


def copy_calibration(torch, nbytes):
    import ctypes
    from decode_gemv_elementwise_amd import build as b
    lib = ctypes.CDLL(b.PROBE_LIB)
    lib.hbm_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
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
        self.bytes_per_step = sum(self.call_bytes(c) for c in self.calls)

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

    def call_bytes(self, c):
        w = self.wl.weights[c.w]
        ops = (1 if c.m else 0) + (1 if c.r else 0)
        w2 = self.wl.weights[c.w2].data.size if c.w2 else 0
        signs = 4 * self.wl.vectors[c.fwht[0]].size if c.fwht else 0
        return w.data.size + w2 + signs + c.ncols * (4 * w.K + 4 * w.N * ops + 4 * w.N)

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


def time_steps(torch, step, steps, warmup, launch):
    """Returns elapsed seconds for `steps` steps after `warmup` untimed ones,
    measured with HIP events on the stream the kernels are launched on."""
    stream = torch.cuda.Stream()
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
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            gt.replay()
            e1.record(stream)
        else:
            run_steps(step, warmup)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            run_steps(step, steps, offset=warmup)
            e1.record(stream)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3


def probe_bandwidth(torch, nbytes=2 << 30):
    import ctypes
    from decode_gemv_elementwise_amd import build as b
    lib = ctypes.CDLL(b.PROBE_LIB)
    lib.hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
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


def read_once_us(torch, nbytes, steps, warmup, store=False):
    """Per-launch time of a kernel that only reads nbytes (one pass, every
    load issued at once), over rotating buffers totalling more than 512 MiB
    and replayed as a graph on its own stream, like the GEMV timing: the
    shortest launch any kernel reading that many bytes can have here.  With
    store, every wave also writes one result at the end, as a GEMV must."""
    import ctypes
    from decode_gemv_elementwise_amd import build as b
    lib = ctypes.CDLL(b.PROBE_LIB)
    fn = lib.hbm_read_once_store if store else lib.hbm_read_once
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.hbm_read_once_blocks.argtypes = [ctypes.c_int64]
    nbytes = (nbytes + 15) // 16 * 16
    slot = (nbytes + 4095) // 4096 * 4096
    copies = max(2, -(-(512 << 20) // slot))
    buf = torch.ones(copies * slot // 4, dtype=torch.float32, device="cuda")
    out = torch.zeros(4 * lib.hbm_read_once_blocks(nbytes), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        s = stream.cuda_stream
        assert fn(buf.data_ptr(), nbytes, out.data_ptr(), s) == 0
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(warmup + steps):
                fn(buf.data_ptr() + (i % copies) * slot, nbytes, out.data_ptr(), s)
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (warmup + steps)
    del g, buf, out
    torch.cuda.empty_cache()
    return us


def cpu_baseline(wl, seconds):
    """The oracle as written (single thread, double precision), on full calls of
    the same workload, for about `seconds` of CPU time."""
    import oracle
    calls = wl.calls
    outputs = {}
    t0 = time.perf_counter()
    nbytes = 0
    ncalls = 0
    while True:
        for c in calls:
            w = wl.weights[c.w]
            x = outputs[c.x[1:]] if c.x.startswith("@") else wl.vectors[c.x]
            m = (outputs[c.m[1:]] if c.m.startswith("@") else wl.vectors[c.m]) if c.m else None
            r = wl.vectors[c.r] if c.r else None
            if c.w2 and c.ncols > 1:
                y = oracle.glu_ncols_reference(w.fmt, w.N, w.K, w.data, wl.weights[c.w2].data,
                                               np.reshape(x, (c.ncols, w.K)), c.act)[0].reshape(-1)
            elif c.w2:
                y = oracle.glu_reference(w.fmt, w.N, w.K, w.data, wl.weights[c.w2].data, x, c.act)[0]
            elif c.fwht:
                y = oracle.fwht_gemv_reference(w.fmt, w.N, w.K, w.data, x, wl.vectors[c.fwht[0]], c.fwht[1], c.act,
                                               m=m, r=r)[0]
            elif c.ncols > 1:
                y = oracle.ncols_reference(w.fmt, w.N, w.K, w.data, np.reshape(x, (c.ncols, w.K)), c.act,
                                           M=m, R=r)[0].reshape(-1)
            else:
                y, _, _ = oracle.reference(w.fmt, w.N, w.K, w.data, x, c.act, m=m, r=r)
            outputs[c.name] = y.astype(np.float32)
            ops = (1 if c.m else 0) + (1 if c.r else 0)
            w2 = wl.weights[c.w2].data.size if c.w2 else 0
            signs = 4 * wl.vectors[c.fwht[0]].size if c.fwht else 0
            nbytes += w.data.size + w2 + signs + c.ncols * (4 * w.K + 4 * w.N * ops + 4 * w.N)
            ncalls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(nbytes / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{ncalls} full calls of {wl.name} (every row, double accumulation, "
                      f"separate epilogue pass) in {el:.1f} s on one host thread",
            "us_per_call": round(el / ncalls * 1e6, 1)}


def cpu_fused_baseline(wl, seconds):
    """The CPU comparison GEMV (tile-fused epilogue, AVX2 vectors, every host
    core) on the same workload's full calls, fused and unfused, for about
    `seconds` of wall time each; None when a call kind has no CPU path."""
    from decode_gemv_elementwise_amd import cpu_fused
    if not cpu_fused.available():
        return None
    if any(c.w2 or c.ncols > 1 or c.fwht for c in wl.calls):
        return None
    threads = len(os.sched_getaffinity(0))
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


def read_counters(workload):
    """Per-launch HBM traffic (bytes) from the committed rocprofv3 counter
    summary of this workload's dominant kernel, if it was taken on the current
    kernel source; else None."""
    path = os.path.join(PROFILES, f"counters_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_sha():
        return None
    try:
        return float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def bench_workload(torch, binding, synth, name, args, probe):
    wl = synth.WORKLOADS[name](0)
    log(f"workload {name}: preparing rotating copies")
    step = Step(torch, binding, wl, args.unfused)
    log(f"  {step.copies} copies, {step.launches_per_step()} launches/step, "
        f"{step.bytes_per_step} algorithmic bytes/step")
    sec = time_steps(torch, step, args.steps, args.warmup, args.launch)
    ms_per_step = sec / args.steps * 1e3
    value = step.bytes_per_step * args.steps / sec / 1e9

    # dominant kernel: the call with the most bytes; timed alone the same way
    dom = max(wl.calls, key=step.call_bytes)
    if len(wl.calls) == 1 and step.launches_per_step() == 1:
        dom_sec = sec / args.steps
    else:
        # inputs produced by earlier calls of the step become fresh vectors of
        # the same length (timing only)
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
        sub = synth.Workload(wl.name, ws, vecs, [alone])
        dstep = Step(torch, binding, sub, False)
        dom_sec = time_steps(torch, dstep, args.steps, args.warmup, args.launch) / args.steps
        del dstep
    dom_bytes = step.call_bytes(dom)
    dom_w = wl.weights[dom.w]
    dom_flops = 2 * dom_w.N * dom_w.K * dom.ncols * (2 if dom.w2 else 1)
    achieved = dom_bytes / dom_sec / 1e9
    cols_kernel = binding.gemv_ncols_kernel(dom_w.fmt, dom_w.N, dom_w.K, dom.ncols) if dom.ncols > 1 else None
    if dom.w2 and dom.ncols > 1:
        kernel_name = (f"gemv_cols_mfma_kernel<{dom_w.fmt}, ncols={dom.ncols}> x2, gated pair as up then gate ({dom.name})"
                       if cols_kernel == "columns_matrix" and dom.act == "silu" else
                       f"gemv_cols(_tiles)_kernel<{dom_w.fmt}, ncols={dom.ncols}, gated pair> ({dom.name})")
    elif cols_kernel == "columns_matrix":
        kernel_name = f"gemv_cols_mfma_kernel<{dom_w.fmt}, ncols={dom.ncols}> ({dom.name})"
    elif dom.ncols > 1:
        kernel_name = f"gemv_cols_kernel<{dom_w.fmt}, ncols={dom.ncols}> ({dom.name})"
    elif dom.fwht:
        kernel_name = f"gemv_fast_kernel<{dom_w.fmt}, signed Hadamard prologue> ({dom.name})"
    else:
        kernel_name = f"gemv_fast_kernel<{dom_w.fmt}{', gated pair' if dom.w2 else ''}> ({dom.name})"
    traffic = read_counters(name)
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
            "launch": args.launch, "rotating_copies": step.copies,
            "algorithmic_bytes_per_step": step.bytes_per_step},
        "us_per_step": round(ms_per_step * 1e3, 3),
        "pct_of_hbm_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "kernel": kernel_name,
                     "algorithmic_bytes_per_launch": dom_bytes,
                     "us_per_launch": round(dom_sec * 1e6, 3)},
    }
    # one FMA per weight and destination column: where that work at the peak
    # of the units that run it (the matrix cores for the matrix-core column
    # kernel, else the vector ALUs) takes longer than the bytes at the HBM
    # peak, the ALU is the roof
    peak_flops = PEAK_MFMA_F16_TFLOPS if cols_kernel == "columns_matrix" else PEAK_VALU_TFLOPS
    if dom_flops / (peak_flops * 1e12) > dom_bytes / (PEAK_HBM_GBPS * 1e9):
        tflops = dom_flops / dom_sec / 1e12
        res["roofline"].update({"bound": "alu", "achieved": round(tflops, 3), "peak": round(PEAK_VALU_TFLOPS, 1),
                                "unit": "TFLOP/s", "frac": round(tflops / PEAK_VALU_TFLOPS, 4),
                                "algorithmic_flops_per_launch": dom_flops,
                                "hbm_gbps": round(achieved, 2)})
    if probe is not None:
        res["probe_read_gbps"] = round(probe, 1)
        res["roofline"]["frac_of_probe"] = round(achieved / probe, 4)
        # the same bytes read by a kernel that does nothing else: what the
        # launch and the stream alone cost at this size
        floor_us = read_once_us(torch, dom_bytes, args.steps, args.warmup)
        res["roofline"]["same_size_read_us"] = round(floor_us, 3)
        res["roofline"]["frac_of_same_size_read"] = round(floor_us / (dom_sec * 1e6), 4)
        # ... and then one store per wave, which every GEMV launch also waits for
        floor_st_us = read_once_us(torch, dom_bytes, args.steps, args.warmup, store=True)
        res["roofline"]["same_size_read_store_us"] = round(floor_st_us, 3)
        res["roofline"]["frac_of_same_size_read_store"] = round(floor_st_us / (dom_sec * 1e6), 4)
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
    if args.steps < 1 or args.warmup < 0:
        sys.exit("steps must be >= 1 and warmup >= 0")
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
    for i, name in enumerate(names):
        res, wl = bench_workload(torch, binding, synth, name, args, probe)
        if i == 0 and args.cpu_seconds > 0:
            log("cpu baseline (oracle)")
            res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
            log("cpu comparison (tile-fused GEMV, all host cores)")
            res["cpu_fused"] = cpu_fused_baseline(wl, args.cpu_seconds / 2)
        print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
