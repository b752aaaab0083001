"""E4M3 query quantization for the indexer (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages keep the KV cache in FP8 (page "Un contexte d'un million sur huit
H200", section "Les chiffres") and say nothing of the indexer's query
precision.  This module defines an optional variant in which the indexer's
queries are also E4M3, so that the q.k contraction runs with both operands in
FP8.  The rule, per (request, position, head) vector q[0..D-1] of bf16 values:

    amax  = max_d |q[d]|                                      (exact)
    if amax < 2^-64:  codes = 0, s = 0                        (zero or negligible head)
    else:          inv   = fl32(448 / amax)                   (binary32 division)
                   x[d]  = fl32(q[d] * inv)                   (binary32 product)
                   codes = nearest E4M3FN value to x[d], ties to the even code
                   s     = fl32(amax / 448)
    w_scaled[h] = fl32(w[h] * s)

fl32 is IEEE binary32 round-to-nearest-even.  The 2^-64 floor keeps 448/amax
finite (bf16 reaches down to 2^-133); a head that small adds at most
128 * 2^-64 * |k| * |w| to a score.  Every step that decides a code
is a binary32 operation, so a binary32 implementation reproduces the codes
exactly.  Because s >= 0, the scale leaves the ReLU:
w * ReLU((s * q8) . k) = (w * s) * ReLU(q8 . k).  The quantized indexer is
therefore the ordinary indexer applied to the E4M3 values of the codes, with
w_scaled as the head weights (``indexer.indexer_scores`` with q_dtype "e4m3").
"""

from __future__ import annotations

import numpy as np

from .numerics import E4M3_MAX, decode_bf16, e4m3fn_table

_TAB = e4m3fn_table()
# non-negative finite values in code order: codes 0x00 .. 0x7E
_POS = _TAB[:0x7F]


def encode_e4m3_rne(x) -> np.ndarray:
    """float32 values -> E4M3FN codes (uint8), nearest value, ties to even.

    The sign bit is copied (a negative value that rounds to zero gives 0x80).
    Magnitudes at or above 464, half-way between 448 and the first value the
    format lacks, have no nearest finite code and are rejected.
    """
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("the encoder takes binary32 values")
    if np.any(np.isnan(x)):
        raise ValueError("NaN has no E4M3 code in this rule")
    mag = np.abs(x.astype(np.float64))                  # exact
    if np.any(mag >= 464.0):
        raise ValueError("magnitude beyond the E4M3 range")
    # the two candidates around each magnitude, by position in the sorted table
    hi = np.searchsorted(_POS, mag, side="left")         # _POS[hi] >= mag
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _POS[lo]
    d_hi = _POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    exact = _POS[hi] == mag
    code = np.where(exact | pick_hi, hi, lo).astype(np.uint8)
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    return code | sign


def quantize_queries(q_bits, w):
    """Per-(b, p, h) E4M3 quantization of bf16 indexer queries.

    q_bits  [..., H, D] uint16 bf16 bit patterns
    w       [..., H]    float32 head weights
    Returns (codes [..., H, D] uint8, w_scaled [..., H] float32, s [..., H] float32).
    """
    q = decode_bf16(q_bits).astype(np.float32)          # exact: bf16 is a binary32 prefix
    w = np.asarray(w, dtype=np.float32)
    amax = np.abs(q).max(axis=-1)                        # [..., H]
    nz = amax >= np.float32(2.0 ** -64)
    safe = np.where(nz, amax, np.float32(1.0))
    inv = (np.float32(E4M3_MAX) / safe).astype(np.float32)
    x = (q * inv[..., None]).astype(np.float32)
    codes = encode_e4m3_rne(x)
    codes = np.where(nz[..., None], codes, np.uint8(0)).astype(np.uint8)
    s = np.where(nz, (safe / np.float32(E4M3_MAX)).astype(np.float32), np.float32(0.0))
    s = s.astype(np.float32)
    w_scaled = (w * s).astype(np.float32)
    return codes, w_scaled, s
