"""Oracle-side decoding of stored weight formats (test infrastructure only).

* BF16: the upper 16 bits of an IEEE binary32; decoding is exact.
* MXFP4 (OCP Microscaling Formats v1.0, the "mxfp4 x mxfp4" MMA kind named in
  [lmsys] "NVFP4 as a third MMA kind", and the MXFP4 checkpoint AMD ships per
  [lmsys] "AMD Support / Day-0 Enablement"): each block of 32 consecutive
  elements along the contiguous (input, K) axis shares one E8M0 scale; each
  element is FP4 E2M1. Stored as two elements per byte, element 2i in the low
  nibble. Value = scale * element, exact in FP64.

* MXFP8 activations (the "fp8 x fp4" MMA kind, [lmsys] "NVFP4 as a third MMA
  kind"; the quantiser that takes the pre-expert norm in [lmsys] "Fuse
  normalization and remove routing conversions"): blocks of 32 consecutive
  elements along the reduction axis share one E8M0 scale; elements are OCP
  FP8 E4M3.

Tables written from the OCP definitions (OCP 8-bit floating point v1.0, OCP MX v1.0):
  E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; exponent 0 is
        subnormal (0 or 0.5). Magnitudes by code 0..7: 0, .5, 1, 1.5, 2, 3, 4, 6.
  E4M3: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0; exponent 0
        is subnormal (m/8 * 2^-6); no infinities; S.1111.111 is NaN, so the
        largest magnitude is 1.75 * 2^8 = 448.
  E8M0: unsigned exponent, value 2^(code-127); code 255 is NaN.
MX quantisation of a block (OCP MX v1.0): X = 2^(floor(log2(amax)) - emax) with
emax the element format's largest exponent (2 for E2M1, 8 for E4M3), each
element v/X rounded to the nearest representable element (ties to the even
code), saturating at the largest magnitude; an all-zero block takes X = 2^-127.
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


def _e4m3_table() -> np.ndarray:
    """Value of each of the 256 E4M3 codes (NaN for the two NaN codes)."""
    vals = np.empty(256, np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 15
        m = code & 7
        if e == 15 and m == 7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3 = _e4m3_table()
E4M3_MAX = 448.0


def _nearest_even(mag: np.ndarray, grid: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Round non-negative magnitudes to the nearest value of an ascending grid
    (codes give each grid value's code; ties go to the even code)."""
    i = np.clip(np.searchsorted(grid, mag), 1, len(grid) - 1)
    lo, hi = grid[i - 1], grid[i]
    dlo, dhi = mag - lo, hi - mag
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (codes[i] % 2 == 0))
    return np.where(pick_hi, hi, lo)


def quantize_mx(v: np.ndarray, fmt: str) -> tuple[np.ndarray, np.ndarray]:
    """MX-quantise v [..., K] (K % 32 == 0) in blocks of 32 along the last axis.
    Returns (dequantised values, scale exponents e with X = 2^e), FP64."""
    if fmt == "mxfp8":
        table, emax, vmax = E4M3[:0x7F], 8, E4M3_MAX  # codes 0..126: +0 .. 448
    elif fmt == "mxfp4":
        table, emax, vmax = E2M1[:8], 2, 6.0
    else:
        raise ValueError(fmt)
    K = v.shape[-1]
    b = v.reshape(v.shape[:-1] + (K // 32, 32))
    amax = np.abs(b).max(-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - emax, -127.0)
    e = np.clip(e, -127.0, 127.0)
    X = np.ldexp(1.0, e.astype(np.int64))[..., None]
    q = b / X
    codes = np.arange(len(table))
    mag = _nearest_even(np.minimum(np.abs(q), vmax), table, codes)
    out = (np.sign(q) * mag * X).reshape(v.shape)
    return out, e


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
