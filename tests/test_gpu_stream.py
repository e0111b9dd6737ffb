"""GPU check of the reference streaming kernels (the bench's measured
bandwidth denominator), through the C ABI: the copy is byte-exact, including
a size that is not a multiple of the grid step, and the read pass's
per-workgroup sums add up to the fp64 sum of the input within fp32
rounding; bad sizes and alignment are rejected on the host."""
import ctypes

import numpy as np
import pytest

from helpers import dev, host

torch = pytest.importorskip("torch")
S = pytest.importorskip("sparse_matrix_vector_amd")

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [4, 1000, 262144 * 4 + 12, 50_000_004])
def test_copy_and_read(n):
    rng = np.random.default_rng(n % 1000)
    a = rng.uniform(-1, 1, n).astype(np.float32)
    src = dev(a)
    dst = torch.full((n,), float("nan"), device="cuda")
    S.spmv_stream_copy(src, dst)
    torch.cuda.synchronize()
    assert np.array_equal(host(dst).view(np.uint32), a.view(np.uint32))
    part = torch.zeros(4096, device="cuda")
    S.spmv_stream_read(src, part)
    torch.cuda.synchronize()
    total = float(host(part).astype(np.float64).sum())
    assert abs(total - a.astype(np.float64).sum()) <= 1e-6 * np.abs(a).sum() + 1e-6


def test_rejects_bad_arguments():
    L = S.lib()
    assert L.spmv_stream_copy(4096, 8192, 20, None) == 1          # not a multiple of 16
    assert L.spmv_stream_copy(4100, 8192, 32, None) == 1          # misaligned source
    assert L.spmv_stream_read(4096, 32, None, 4096, None) == 1    # no partial buffer
    assert L.spmv_stream_read(4096, 1 << 20, 8192, 16, None) == 1  # fewer partials than workgroups
    assert L.spmv_stream_copy(None, None, 0, None) == 0           # nothing to do
