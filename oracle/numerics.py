"""Rounding of the step's API-visible tensors to their storage precision.

The pages fix no precision.  Reading taken: the tensors the step hands from
one stage to the next (X, Q, K_new, V_new, O, Z, S) are stored in the
workload's storage type (bfloat16 or float32); the oracle mirrors exactly
that storage and computes in float64 everywhere else.
"""
import numpy as np


def round_bf16(x):
    """float64 -> nearest bfloat16 value (ties to even), returned as float64.
    bfloat16 keeps 8 significant bits and float32's exponent range; frexp
    puts the significand in [0.5, 1), so rounding significand*256 to an
    integer (np.round: half to even) keeps exactly 8 bits."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.round(m * 256.0) / 256.0, e)


def round_store(x, dtype):
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(dtype)
