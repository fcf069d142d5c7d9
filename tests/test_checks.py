"""The GPU tests' full-size checking helpers, run on the CPU against planted mistakes: an exact
product passes; one wrong entry, two swapped entries, a wrong row and a transposed block fail.
Integer operands keep every partial sum exact (see _freivalds_exact)."""
import numpy as np
import pytest

from tests.test_gpu_gemm import _freivalds_exact, _int_operands


@pytest.mark.parametrize("bl", ["kn", "nk"])
@pytest.mark.parametrize("sparse", [True, False])
def test_freivalds_catches_planted_errors(bl, sparse):
    rng = np.random.default_rng(5)
    M, N, K = 96, 80, 64
    A, B = _int_operands(rng, M, N, K, bl, sparse)
    Bkn = B if bl == "kn" else B.T
    C = (A.astype(np.int64) @ Bkn.astype(np.int64)).astype(np.float32)
    if sparse:
        assert np.abs(C).max() <= 256
    _freivalds_exact(C, A, B, bl, 1, "exact")
    bad = C.copy()
    bad[17, 33] += 1
    with pytest.raises(AssertionError):
        _freivalds_exact(bad, A, B, bl, 1, "one entry")
    bad = C.copy()
    bad[5, [3, 40]] = bad[5, [40, 3]] + np.array([1.0, -1.0])  # swapped, and different
    with pytest.raises(AssertionError):
        _freivalds_exact(bad, A, B, bl, 1, "swapped pair")
    bad = C.copy()
    bad[60] = bad[61]
    if not np.array_equal(C[60], C[61]):
        with pytest.raises(AssertionError):
            _freivalds_exact(bad, A, B, bl, 1, "wrong row")
    bad = C.copy()
    bad[:16, :16] = bad[:16, :16].T.copy()
    if not np.array_equal(C[:16, :16], C[:16, :16].T):
        with pytest.raises(AssertionError):
            _freivalds_exact(bad, A, B, bl, 1, "transposed block")
