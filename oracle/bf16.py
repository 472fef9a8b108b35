"""bfloat16 rounding emulation (oracle; test infrastructure only).

bfloat16 keeps float32's 8-bit exponent and 8 significant bits (7 stored
fraction bits). The decoder's bf16 workloads store the query projection Q
and the key/value projections K, V in bf16; the oracle reproduces that
rounding point from its exact (float64) values with this function, so that
it rounds once, directly from float64, to nearest with ties to even.
"""

import numpy as np


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even).

    The quantum at x = m * 2**e (0.5 <= |m| < 1) is 2**(e - 8) for normal
    numbers and 2**-133 below 2**-126 (subnormal range). Values beyond the
    largest finite bf16 become +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    _, e = np.frexp(x[nz])
    q = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.rint(x[nz] / q) * q  # np.rint rounds half to even
    big = np.abs(r) > 3.3895313892515355e38  # largest finite bf16
    r[big] = np.copysign(np.inf, r[big])
    out[nz] = r
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out
