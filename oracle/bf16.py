"""bf16 storage conversions for the oracle (test infrastructure only).

The FastFlowLM card ("Weights" row of its spec table) stores norms, the
dynamic-convolution tensors, the selector projection and codebooks in BF16, and
its "Measured draft quality" table runs the draft with bf16 activations.  A bf16
value is the top 16 bits of an IEEE float32; widening is exact.
"""
import numpy as np


def bf16_to_f64(u16):
    """uint16 bf16 bit patterns -> float64 (exact)."""
    u16 = np.asarray(u16, dtype=np.uint16)
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16(x):
    """float64 -> bf16 bit patterns, round to nearest, ties to even.

    Rounds directly from the float64 value (not via float32), so the result is
    the bf16 value nearest to x.  Finite inputs only.
    """
    x = np.asarray(x, dtype=np.float64)
    # bf16 keeps 8 significant bits.  Scale each value so that its leading bit
    # sits at 2^7, round to an integer with ties-to-even, scale back.
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    r = np.rint(m * 256.0) / 256.0          # 8 significant bits, RNE
    y = np.ldexp(r, e).astype(np.float32)   # exact: y has <= 8 significant bits
    bits = y.view(np.uint32)
    return (bits >> 16).astype(np.uint16)


def round_bf16(x):
    """float64 -> nearest bf16 value, returned as float64."""
    return bf16_to_f64(f64_to_bf16(x))
