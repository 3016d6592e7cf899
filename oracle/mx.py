"""Oracle-side decoding of stored weight formats (test infrastructure only).

* BF16: the upper 16 bits of an IEEE binary32; decoding is exact.
* MXFP4 (OCP Microscaling Formats v1.0, the "mxfp4 x mxfp4" MMA kind named in
  [lmsys] "NVFP4 as a third MMA kind", and the MXFP4 checkpoint AMD ships per
  [lmsys] "AMD Support / Day-0 Enablement"): each block of 32 consecutive
  elements along the contiguous (input, K) axis shares one E8M0 scale; each
  element is FP4 E2M1. Stored as two elements per byte, element 2i in the low
  nibble. Value = scale * element, exact in FP64.

Tables written from the OCP MX v1.0 definitions:
  E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; exponent 0 is
        subnormal (0 or 0.5). Magnitudes by code 0..7: 0, .5, 1, 1.5, 2, 3, 4, 6.
  E8M0: unsigned exponent, value 2^(code-127); code 255 is NaN.
"""
from __future__ import annotations

import numpy as np


def _e2m1_table() -> np.ndarray:
    vals = np.empty(16, np.float64)
    for code in range(16):
        sign = -1.0 if code & 8 else 1.0
        e = (code >> 1) & 3
        m = code & 1
        if e == 0:
            mag = 0.5 * m  # subnormal: 2^(1-bias) * (m/2) with bias 1
        else:
            mag = 2.0 ** (e - 1) * (1.0 + 0.5 * m)
        vals[code] = sign * mag
    return vals


E2M1 = _e2m1_table()


def e8m0_to_f64(codes: np.ndarray) -> np.ndarray:
    c = codes.astype(np.int64)
    out = np.ldexp(1.0, c - 127).astype(np.float64)
    out[c == 255] = np.nan
    return out


def bf16_to_f64(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def mxfp4_to_f64(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """packed [..., K/2] uint8, scales [..., K/32] uint8 -> float64 [..., K]."""
    lo = packed & 0x0F
    hi = packed >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(packed.shape[:-1] + (packed.shape[-1] * 2,))
    elems = E2M1[codes]
    K = elems.shape[-1]
    s = e8m0_to_f64(scales)
    return (elems.reshape(elems.shape[:-1] + (K // 32, 32)) * s[..., None]).reshape(elems.shape)


def to_f64(a) -> np.ndarray:
    """Decode any stored tensor (float32 array, uint16 BF16 bits, or an MXFP4
    (packed, scales) pair) to float64."""
    if isinstance(a, tuple):
        return mxfp4_to_f64(*a)
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    return a.astype(np.float64)
