"""Error measures used by the GPU parity tests.

The bar: max|got - ref| / rms(ref) <= 1e-4 for fp32 q/k/v and <= 3e-3 for
bf16 q/k/v with fp32 gates and state, applied to the outputs o and to the
final states alike (the state measure uses the state's own rms).
"""
import numpy as np

TOL_FP32 = 1e-4
TOL_BF16 = 3e-3


def rel_max_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = float(np.max(np.abs(got - ref)))
    if rms == 0.0:
        return err
    return err / rms


def tol_for(dtype):
    return TOL_FP32 if dtype == "fp32" else TOL_BF16
