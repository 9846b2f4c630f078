"""Exact decoding of the storage formats the library consumes (oracle side).

bf16: the upper 16 bits of an IEEE-754 binary32; decoding is exact.
fp8 e4m3fn (OCP 8-bit floating point specification, E4M3 variant): 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
subnormals m/8 * 2^-6; there is no infinity; S.1111.111 is NaN; the largest
finite magnitude is 1.75 * 2^8 = 448.  The DSA indexer runs in "FP8
arithmetic" ([IC-SUMMARY] §2.1); e4m3fn is the reading taken for it.
"""
import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _e4m3fn_table() -> np.ndarray:
    tab = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            tab[code] = np.nan
        elif e == 0:
            tab[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            tab[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return tab


E4M3FN = _e4m3fn_table()


def e4m3fn_codes_to_f64(codes) -> np.ndarray:
    """uint8 e4m3fn codes -> float64 (exact)."""
    return E4M3FN[np.asarray(codes).astype(np.uint8)]


def dequantize(raw, dtype: str, scale=None) -> np.ndarray:
    """Raw storage -> float64.  ``dtype`` is 'f32' (float32 array), 'bf16'
    (uint16 bit patterns) or 'fp8' (uint8 e4m3fn codes).  ``scale`` (fp32),
    if given, multiplies every vector along the last axis: x = scale * code,
    the product taken exactly in float64."""
    if dtype == "f32":
        x = np.asarray(raw, dtype=np.float32).astype(np.float64)
    elif dtype == "bf16":
        x = bf16_bits_to_f64(raw)
    elif dtype == "fp8":
        x = e4m3fn_codes_to_f64(raw)
    else:
        raise ValueError(dtype)
    if scale is not None:
        x = x * np.asarray(scale, dtype=np.float32).astype(np.float64)[..., None]
    return x
