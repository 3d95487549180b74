"""FP8 E4M3 ("e4m3fn") codes -> values, written from the format's definition.

TEST INFRASTRUCTURE (see the package docstring). Follows the E4M3 format that the
FastUSP page (mlsanity) builds on ("FP8 Formats for Deep Learning", in its list of
prior work): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits. Exponent
field 0 encodes subnormals m/8 * 2^-6; the all-ones exponent with all-ones mantissa
is NaN and there are no infinities, so the largest finite magnitude is
1.75 * 2^8 = 448. A code of batch b and head h stands for decode(code) * scale[b, h].
An fp8 attention state stores its OUT as codes with one factor per row (the FastUSP
page's FP8-quantised attention traffic, applied to states): element (r, d) stands for
decode(code[r, d]) * factor[r].
"""
from __future__ import annotations

import numpy as np

BIAS = 7


def decode_e4m3(codes) -> np.ndarray:
    """Value of each uint8 code, as float64 (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2((e - BIAS).astype(np.float64))
    subnormal = (m / 8.0) * np.exp2(1.0 - BIAS)
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, mag)
    return sign * mag


def dequantize(codes, scale) -> np.ndarray:
    """codes [B, H, S, D] (uint8) and scale [B, H] -> float64 values decode(code) * scale[b, h]."""
    vals = decode_e4m3(codes)
    s = np.asarray(scale, dtype=np.float64)
    return vals * s[:, :, None, None]


def decode_state(codes, factors) -> np.ndarray:
    """An fp8 state's OUT: codes [..., rows, D] (uint8) and row factors [..., rows] -> float64
    decode(code) * factor of the code's row."""
    return decode_e4m3(codes) * np.asarray(factors, dtype=np.float64)[..., None]
