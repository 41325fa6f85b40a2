"""bfloat16 rounding emulation on bit patterns (oracle side).

bfloat16 keeps the float32 exponent and the top 7 stored mantissa bits. A
value is rounded to nearest, ties to even. The oracle rounds a float64 value
first to float32 (the format every float32 intermediate of the method is held
in) and then to bfloat16, as a float32 producer storing bfloat16 does.
"""
import numpy as np


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    return ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16 rounding of a non-finite value")
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float64).astype(np.float32))


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 and return the exact value as float64."""
    return bf16_bits_to_f64(f64_to_bf16_bits(x))
