"""Number formats of the inputs, decoded to float64 from their definitions.

bf16: the upper 16 bits of an IEEE-754 binary32, so decoding is a shift.

e4m3fn (OCP 8-bit floating point, E4M3 "fn" variant: 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits, no infinities, only S.1111.111 is NaN):
  exponent field e > 0 : (-1)^s * (1 + m/8) * 2^(e - 7)
  exponent field e = 0 : (-1)^s * (m/8) * 2^(-6)          (subnormal)
The largest finite value is S.1111.110 = 448.

The pages name the keys only as fp8; which fp8 variant is a reading (the OCP
fn variant, the one gfx950 converts natively).
"""
import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def _e4m3fn_value(code: int) -> float:
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float('nan')
    if e == 0:
        mag = (m / 8.0) * 2.0 ** (-6)
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def e4m3fn_table() -> np.ndarray:
    """The 256 code values as float64 (index = code)."""
    return np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


_TABLE = e4m3fn_table()


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """e4m3fn bit patterns (uint8) -> float64, exactly."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]
