"""Value decoding for the oracle (test infrastructure only)."""

import numpy as np


def as_f64(x):
    """Exact float64 values of an input tensor.

    uint16 arrays are bf16 bit patterns (the top half of a float32); float32
    and float64 arrays are taken as they are.
    """
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError("unsupported input dtype %s" % a.dtype)
