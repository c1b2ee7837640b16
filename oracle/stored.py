"""Stored values -> float64, and float64 -> nearest bf16 value.  (Oracle: test infrastructure.)

bf16 arrays arrive as their uint16 bit patterns; the value is the float32 whose high
half is those bits, which float64 holds exactly.
"""
import numpy as np


def to_f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported stored dtype {a.dtype}")


def round_bf16(x) -> np.ndarray:
    """Nearest bf16 value (8 significant bits, ties to even) of float64 x, as float64.

    Written with frexp/rint: x = m * 2^e, 0.5 <= |m| < 1; keep 8 significant bits of m.
    np.rint rounds half to even.  Normal range only (|x| well inside bf16's range)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def to_bf16_bits(x) -> np.ndarray:
    """Stored bf16 bit patterns (uint16) of float64 values that are already bf16 values
    (e.g. the output of round_bf16): the float32 of such a value is exact, and its upper
    half is the pattern."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if not np.array_equal(x32.astype(np.float64), np.asarray(x, dtype=np.float64)):
        raise ValueError("to_bf16_bits: value is not a bf16 value")
    bits = x32.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("to_bf16_bits: value is not a bf16 value")
    return (bits >> 16).astype(np.uint16)
