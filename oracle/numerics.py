"""Number formats used by the KV caches and queries (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Both deployments on the page "Un contexte d'un million sur huit H200"
(section "Les chiffres") keep the KV cache in FP8.  The pages do not name the
FP8 variant; the reading taken is OCP FP8 E4M3FN ("fn": finite, no infinity),
the format gfx950 converts natively.  The table below is built from the
format's definition, field by field, and is pinned against torch's own
``float8_e4m3fn`` conversion and against hand-decoded codes in the tests.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3fn_value(code: int) -> float:
    """Value of one E4M3FN byte, from the OCP FP8 field definition.

    sign s (bit 7), exponent e (bits 6..3, bias 7), mantissa m (bits 2..0):
      e == 0          -> (-1)^s * 2^-6 * (m / 8)        (subnormal, incl. +-0)
      e == 15, m == 7 -> NaN                            (0x7F and 0xFF)
      otherwise       -> (-1)^s * 2^(e - 7) * (1 + m/8)
    There is no infinity; the largest finite magnitude is 2^8 * 1.75 = 448.
    """
    code = int(code) & 0xFF
    s = code >> 7
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = 2.0 ** -6 * (m / 8.0)
    else:
        mag = 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -mag if s else mag


def e4m3fn_table() -> np.ndarray:
    """float64[256]: value of every E4M3FN code."""
    return np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


_E4M3_TABLE = e4m3fn_table()


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values (same shape)."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("E4M3 codes must be uint8")
    return _E4M3_TABLE[codes]


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64.

    A bfloat16 is the upper half of an IEEE binary32, so placing the 16 bits
    in the top of a 32-bit word gives the same value exactly.
    """
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("bf16 values are passed as their uint16 bit patterns")
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Values of an input array given its storage tag: 'f32', 'bf16' or 'e4m3'."""
    if dtype == "f32":
        x = np.asarray(x)
        if x.dtype != np.float32:
            raise TypeError("f32 input must be float32")
        return x.astype(np.float64)
    if dtype == "bf16":
        return decode_bf16(x)
    if dtype == "e4m3":
        return decode_e4m3(x)
    raise ValueError(f"unknown dtype tag {dtype!r}")
