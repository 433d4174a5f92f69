"""The Python binding refuses, before any library call, torch tensors that a
launch would turn into bad device accesses: host tensors, wrong dtypes,
non-contiguous buffers and buffers shorter than what the kernel reads.  CPU
only: every case raises before anything reaches the GPU."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from decode_gemv_elementwise_amd import binding


@pytest.fixture(scope="module", autouse=True)
def lib():
    try:
        binding.load()
    except ImportError as e:  # pragma: no cover - the build step makes it
        pytest.skip(str(e))


def _w(fmt, N, K, short=0):
    nbytes = binding.gemv_weight_bytes(fmt, N, K) - short
    return torch.zeros(nbytes, dtype=torch.uint8)


def test_host_tensors_are_refused():
    W, x, dst = _w("f16", 8, 64), torch.zeros(64), torch.zeros(8)
    with pytest.raises(TypeError, match="GPU"):
        binding.gemv_fused(W, "f16", 8, 64, x, "none", dst=dst)
    with pytest.raises(TypeError, match="GPU"):
        binding.gemv_glu(W, W, "f16", 8, 64, x, "silu", dst=dst)
    with pytest.raises(TypeError, match="GPU"):
        binding.gemv_fused_ncols(W, "f16", 8, 64, 2, torch.zeros(128), "none", dst=torch.zeros(2, 8))
    with pytest.raises(TypeError, match="GPU"):
        binding.gemv_epilogue("add", 8, torch.zeros(8), add_operand=torch.zeros(8), dst=dst)
    with pytest.raises(TypeError, match="GPU"):
        binding.gemv_fwht_signed(torch.zeros(64), torch.ones(64), 1, 64, 64, 64, torch.zeros(64))
    with pytest.raises(TypeError, match="GPU"):
        binding.PreparedCall(W, "f16", 8, 64, x, "none", dst=dst)


def test_wrong_dtype_is_refused():
    W = _w("f32", 8, 64)
    with pytest.raises(TypeError, match="x must be torch.float32"):
        binding.gemv_fused(W, "f32", 8, 64, torch.zeros(64, dtype=torch.float16), "none", dst=torch.zeros(8))
    with pytest.raises(TypeError, match="acc must be torch.float32"):
        binding.gemv_epilogue("none", 8, torch.zeros(8, dtype=torch.float64), dst=torch.zeros(8))
    with pytest.raises(TypeError, match="signs must be torch.float32"):
        binding.gemv_fwht_signed(torch.zeros(64), torch.ones(64, dtype=torch.int32), 1, 64, 64, 64, torch.zeros(64))
    with pytest.raises(TypeError, match="float32"):
        binding.gemv_fused(W, "f32", 8, 64, torch.zeros(64), "none", dst=torch.zeros(8, dtype=torch.float16))
    with pytest.raises(TypeError, match="x must be torch.float32"):
        binding.gemv_fused_fwht(W, "f32", 8, 64, torch.zeros(64, dtype=torch.float64), torch.ones(64), 64, 64, "none",
                                dst=torch.zeros(8))


def test_short_buffers_are_refused():
    with pytest.raises(ValueError, match="W holds"):
        binding.gemv_fused(_w("q4b32", 16, 256, short=2), "q4b32", 16, 256, torch.zeros(256), "none",
                           dst=torch.zeros(16))
    with pytest.raises(ValueError, match="W_up holds"):
        binding.gemv_glu(_w("q8b32", 16, 256), _w("q8b32", 16, 256, short=1), "q8b32", 16, 256,
                         torch.zeros(256), "silu", dst=torch.zeros(16))
    with pytest.raises(ValueError, match="x holds"):
        binding.gemv_fused(_w("bf16", 16, 256), "bf16", 16, 256, torch.zeros(255), "none", dst=torch.zeros(16))
    with pytest.raises(ValueError, match="x holds"):
        binding.gemv_fused_ncols(_w("f16", 16, 64), "f16", 16, 64, 3, torch.zeros(2, 64), "none",
                                 dst=torch.zeros(3, 16))
    with pytest.raises(ValueError, match="signs holds"):
        binding.gemv_fwht_signed(torch.zeros(2, 64), torch.ones(31), 2, 64, 32, 32, torch.zeros(2, 64))
    with pytest.raises(ValueError, match="dst holds"):
        binding.gemv_fwht_signed(torch.zeros(2, 64), torch.ones(32), 2, 64, 32, 32, torch.zeros(64))
    with pytest.raises(ValueError, match="acc holds"):
        binding.gemv_epilogue("none", 8, torch.zeros(7), dst=torch.zeros(8))


def test_non_contiguous_inputs_are_refused():
    W = _w("f32", 8, 64)
    with pytest.raises(TypeError, match="x must be contiguous"):
        binding.gemv_fused(W, "f32", 8, 64, torch.zeros(128)[::2], "none", dst=torch.zeros(8))
    Wb = torch.zeros(2 * W.numel(), dtype=torch.uint8)[::2]
    with pytest.raises(TypeError, match="W must be contiguous"):
        binding.gemv_fused(Wb, "f32", 8, 64, torch.zeros(64), "none", dst=torch.zeros(8))


def test_host_only_checks_still_take_host_tensors_and_addresses():
    """The *_validate calls make no HIP call, so they keep accepting host
    memory (the library checks shapes, formats and overlaps only)."""
    W, x = _w("f16", 8, 64), torch.zeros(64)
    assert binding.gemv_validate(W, "f16", 8, 64, x, "none", dst=torch.zeros(8)) == 0
    assert binding.gemv_validate(W.data_ptr(), "f16", 8, 64, x.data_ptr(), "none",
                                 dst=binding.make_view(torch.zeros(8))) == 0


def test_rejected_column_counts_reach_the_library_checks():
    """Where the library itself rejects the call (a column count outside
    1..8), the binding does not pre-empt its status with a size error."""
    W, dst = _w("f16", 8, 64), torch.zeros(9, 8)
    with pytest.raises(TypeError, match="GPU"):
        binding.gemv_fused_ncols(W, "f16", 8, 64, 9, torch.zeros(2, 64), "none", dst=dst)
    assert binding.gemv_fused_ncols_validate(W, "f16", 8, 64, 9, torch.zeros(9, 64), "none", dst=dst) == \
        binding.STATUS_CODE["GEMV_E_DIM"]
