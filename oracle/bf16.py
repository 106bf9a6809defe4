"""bfloat16 rounding in float64 (test infrastructure only; see package header).

bfloat16 keeps 8 significant bits (1 implicit + 7 stored) and float32's
exponent range.  Rounding is to nearest, ties to even, taken directly from the
float64 value, so there is no double rounding through float32.
"""
import numpy as np


def to_f64(t):
    """A torch tensor (any float dtype, CPU) as a float64 numpy array, exactly."""
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value (ties to even).

    x = m * 2**e with 0.5 <= |m| < 1; scaling by 2**(8-e) puts the kept bits
    left of the binary point, ``np.rint`` rounds half to even, and scaling
    back is exact.  Below bfloat16's smallest normal (2**-126) the grid
    spacing stays 2**-133, hence the clamp of e at -125.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    xs = x[fin]
    _, e = np.frexp(xs)
    e = np.maximum(e, -125)
    out[fin] = np.ldexp(np.rint(np.ldexp(xs, 8 - e)), e - 8)
    return out
