"""Host logic of bench.py, on the CPU: the algorithmic bytes it charges each
call, the summaries it trusts, and its refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from decode_gemv_elementwise_amd import synth  # noqa: E402

# Algorithmic bytes per call of the five decode configurations: W in its
# storage format + 4K (x) + 4N per epilogue operand read + 4N (dst), worked
# out by hand from their shapes (f32 4 B, f16/bf16 2 B, 8-bit 1 + 2/32 B,
# 4-bit 1/2 + 2/32 B per weight).
EXPECTED = {
    "f32_tiny_256": {"f32_256_none": 264_192, "f32_256_sigmoid": 264_192, "f32_256_silu": 264_192,
                     "f32_256_silu_mul": 265_216, "f32_256_add": 265_216, "f32_256_mul": 265_216},
    "f16_outproj_residual_4096": {"f16_outproj_add_inplace": 33_603_584},
    "bf16_swiglu_gate_14336x4096": {"bf16_swiglu_silu_mul": 117_571_584, "bf16_gate_sigmoid_32": 278_656},
    "q8b32_view_residual_4096x6144": {"q8b32_add_view_32x128": 26_796_032},
    "q4b32_decode_layer": {"q4_qkv_none": 14_196_736, "q4_o_add": 9_486_336, "q4_gate_silu": 33_103_872,
                           "q4_up_mul": 33_161_216, "q4_down_add": 33_120_256, "q4_gate_sigmoid_32": 90_240},
}


@pytest.mark.parametrize("name", sorted(EXPECTED))
def test_algorithmic_bytes_per_call(name):
    wl = synth.WORKLOADS[name](0)
    got = {c.name: bench.call_bytes(wl, c) for c in wl.calls}
    assert got == EXPECTED[name]


def test_layer_step_bytes():
    wl = synth.WORKLOADS["q4b32_decode_layer"](0)
    assert sum(bench.call_bytes(wl, c) for c in wl.calls) == 123_158_656


def _summary(tmp_path, name, sha, body):
    path = tmp_path / name
    path.write_text(f"# a summary\nkernel_source_sha256: {sha}\n{body}")
    return path


def test_summaries_are_used_only_for_the_current_kernel_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    sha = bench.kernel_sha()
    _summary(tmp_path, "counters_w.txt", sha, "fetch_bytes_per_launch: 1000\nwrite_bytes_per_launch: 24\n")
    _summary(tmp_path, "trace_w.txt", sha,
             "dominant_kernel_avg_ns: 8250.0\ntrace_read_store_floor_avg_ns: 6500.0  (median 6400.0, 9 dispatches)\n")
    assert bench.read_counters("w") == 1024.0
    assert bench.read_trace("w") == (8.25, 6.5)
    _summary(tmp_path, "counters_w.txt", "0" * 64, "fetch_bytes_per_launch: 1000\nwrite_bytes_per_launch: 24\n")
    _summary(tmp_path, "trace_w.txt", "0" * 64, "dominant_kernel_avg_ns: 8250.0\n")
    assert bench.read_counters("w") is None
    assert bench.read_trace("w") == (None, None)
    assert bench.read_counters("absent") is None


def test_kernel_sha_covers_every_device_source():
    csrc = os.path.join(ROOT, "decode_gemv_elementwise_amd", "csrc")
    device = {f for f in os.listdir(csrc) if f.endswith((".hip", ".h")) and f not in ("hbm_probe.hip", "gemv_internal.h")}
    assert device == {os.path.basename(p) for p in bench.KERNEL_SOURCES}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
