"""Comparison helpers shared by the tests (no method arithmetic here)."""
import numpy as np


def bf16_ordered(bits: np.ndarray) -> np.ndarray:
    """Map bf16 bit patterns to integers in numeric order (+0 and -0 both map to 0)."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Number of bf16 steps between two bf16 values (0 = equal, 1 = adjacent)."""
    return np.abs(bf16_ordered(a_bits) - bf16_ordered(b_bits))


def fp32_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of float32 at |x|."""
    x = np.abs(np.asarray(x, dtype=np.float32))
    return np.spacing(x).astype(np.float64)
