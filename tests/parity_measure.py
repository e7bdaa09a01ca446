"""The parity measure: max |gpu - oracle| / rms(oracle) over a whole tensor.

rel_err() takes two whole tensors; WholeTensorError feeds a tensor in pieces
(groups of heads, blocks of rows) and gives the same value, so that a
full-size workload can be compared while host memory holds one piece at a
time.  The rms is that of the oracle's tensor; a GPU value that is not finite
fails the comparison outright.
"""
import numpy as np


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "non-finite GPU output"
    rms = float(np.sqrt(np.mean(ref ** 2)))
    diff = float(np.max(np.abs(gpu - ref))) if gpu.size else 0.0
    return diff / rms if rms > 0 else diff


class WholeTensorError:
    """rel_err() of a tensor given piece by piece.

    The running maximum of |gpu - oracle| and the running sum of oracle**2
    over the pieces give rel_err() of their concatenation.
    """

    def __init__(self):
        self.max_diff, self.sum_sq, self.count = 0.0, 0.0, 0

    def add(self, gpu, ref, rows=1 << 20):
        gpu = np.asarray(gpu).reshape(-1)
        ref = np.asarray(ref).reshape(-1)
        assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
        for i in range(0, gpu.size, rows):
            g = gpu[i:i + rows].astype(np.float64)
            r = ref[i:i + rows].astype(np.float64)
            assert np.all(np.isfinite(g)), "non-finite GPU output"
            self.max_diff = max(self.max_diff, float(np.max(np.abs(g - r))))
            self.sum_sq += float(np.dot(r, r))
        self.count += gpu.size
        return self

    def value(self):
        rms = (self.sum_sq / self.count) ** 0.5 if self.count else 0.0
        return self.max_diff / rms if rms > 0 else self.max_diff
