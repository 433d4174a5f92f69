"""Build step: compiles the HIP library ``libgemv_fused.so`` for gfx950 in-tree.

hipcc cross-compiles without a GPU.  Flags:
  -ffp-contract=off     every multiply-add in the kernels is an explicit fmaf,
                        nothing else may be contracted (fused and unfused
                        paths must round identically);
  -packed-fp32-ops off  no packed FP32 instructions are generated.
"""
import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgemv_fused.so")
PROBE_LIB = os.path.join(HERE, "libhbm_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = [os.path.join(CSRC, "gemv_kernels.hip"), os.path.join(CSRC, "gemv_cols.hip"),
           os.path.join(CSRC, "gemv_validate.cpp"), os.path.join(CSRC, "gemv_fwht.hip"),
           os.path.join(CSRC, "gemv_mfma.hip")]
PROBE_SOURCES = [os.path.join(CSRC, "hbm_probe.hip")]
CPU_SOURCE = os.path.join(HERE, "cpu", "cpu_fused.c")
CPU_LIB = os.path.join(HERE, "libcpu_fused.so")
# the CPU comparison GEMV: AVX2 + FMA + F16C hosts
CPU_FLAGS = ["-O3", "-std=c11", "-fPIC", "-shared", "-pthread", "-mavx2", "-mfma", "-mf16c", "-ffp-contract=fast",
             "-Wall"]

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-result"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}):\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")


def _compile(sources, out, verbose):
    """Compiles each source to an object (in parallel), then links them."""
    with tempfile.TemporaryDirectory(prefix="gemv_build_") as tmpdir:
        objs = [os.path.join(tmpdir, f"{i}_{os.path.basename(src)}.o") for i, src in enumerate(sources)]
        cmds = [[HIPCC, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", "-o", o, src]
                for src, o in zip(sources, objs)]
        with ThreadPoolExecutor(max(1, min(len(cmds), 4))) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        tmp = out + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", "-o", tmp, *objs], verbose)
        os.replace(tmp, out)
    return out


def build_cpu(verbose: bool = False) -> str:
    tmp = CPU_LIB + ".tmp"
    _run(["gcc", *CPU_FLAGS, "-I", INCLUDE, "-o", tmp, CPU_SOURCE, "-lm"], verbose)
    os.replace(tmp, CPU_LIB)
    return CPU_LIB


def build(verbose: bool = False) -> str:
    """Builds the GEMV library, the benchmark's measurement library and the
    CPU comparison GEMV."""
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    build_cpu(verbose)
    return _compile(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
