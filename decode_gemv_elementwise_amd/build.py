"""Build step: compiles the HIP library ``libgemv_fused.so`` for gfx950 in-tree.

hipcc cross-compiles without a GPU.  Flags:
  -ffp-contract=off     every multiply-add in the kernels is an explicit fmaf,
                        nothing else may be contracted (fused and unfused
                        paths must round identically);
  -packed-fp32-ops off  no packed FP32 instructions are generated.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgemv_fused.so")
PROBE_LIB = os.path.join(HERE, "libhbm_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = [os.path.join(CSRC, "gemv_kernels.hip"), os.path.join(CSRC, "gemv_validate.cpp")]
PROBE_SOURCES = [os.path.join(CSRC, "hbm_probe.hip")]

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-result"]


def _compile(sources, out, verbose, extra_flags=()):
    tmp = out + ".tmp"
    cmd = [HIPCC, *HIP_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-shared", "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, out: str = LIB, extra_flags=()) -> str:
    """Builds the GEMV library and the benchmark's measurement library."""
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    return _compile(SOURCES, out, verbose, extra_flags)


if __name__ == "__main__":
    print(build(verbose=True))
