"""Number formats of the stored model, written from their bit definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

bf16: the upper 16 bits of an IEEE-754 binary32 (1 sign, 8 exponent, 7
mantissa bits).  Decoding shifts the bits into a binary32, which is exact.
Encoding rounds to nearest, ties to even (the pages fix no rounding; RNE is
the reading used throughout).

E4M3: the 8-bit format of Micikevicius et al., "FP8 Formats for Deep
Learning" (reference list of the kernel-fusion architecture study): 1 sign,
4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds
subnormals m * 2^-9; the all-ones pattern S.1111.111 is NaN; there are no
infinities, so the largest finite magnitude is 1.75 * 2^8 = 448.  Encoding
rounds to nearest-even and saturates finite values to +-448 (never NaN).

int8: two's complement, bit 7 the sign: a byte b >= 128 stands for b - 256.
The weight-only INT8 format of the stored models (per-row scale, symmetric
codes -127..127) is a scale times this integer.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


# ------------------------------------------------------------------ bf16

def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), as float64.

    Works on the float64 value directly (no detour through binary32, which
    could round twice): for |x| in [2^e, 2^(e+1)) the bf16 spacing is 2^(e-7),
    and below 2^-126 it is the subnormal spacing 2^-133.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    ax = np.abs(x[nz])
    _, e2 = np.frexp(ax)  # ax = f * 2^e2, f in [0.5, 1)  ->  exponent e = e2 - 1
    e = np.maximum(e2 - 1, -126)
    q = np.ldexp(1.0, e - 7)
    r = np.rint(ax / q) * q  # rint rounds half to even
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    out[nz] = np.copysign(r, x[nz])
    keep = (x == 0) | ~np.isfinite(x)  # signed zeros, infinities and NaN pass through
    out[keep] = x[keep]
    return out


def bf16_encode(x: np.ndarray) -> np.ndarray:
    """float64 -> uint16 bf16 bits, RNE.  The rounded value is exact in binary32."""
    r = bf16_round(x).astype(np.float32)
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ------------------------------------------------------------------ E4M3

def _e4m3_value(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 E4M3 codes -> float64 values."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest E4M3 value (ties to even, saturating)."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.minimum(np.abs(x), E4M3_MAX)
    out = np.zeros_like(x)
    nz = ax > 0
    _, e2 = np.frexp(ax[nz])
    e = np.maximum(e2 - 1, -6)  # below 2^-6 the spacing is the subnormal 2^-9
    q = np.ldexp(1.0, e - 3)
    r = np.minimum(np.rint(ax[nz] / q) * q, E4M3_MAX)
    out[nz] = r
    return np.copysign(out, x)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float64 -> uint8 E4M3 codes (RNE, saturating; -0.0 keeps its sign bit)."""
    r = e4m3_round(x)
    ar = np.abs(r)
    code = np.zeros(r.shape, dtype=np.uint8)
    sub = ar < 2.0 ** -6
    code[sub] = np.rint(ar[sub] * 2.0 ** 9).astype(np.uint8)
    nrm = ~sub
    if np.any(nrm):
        f, e2 = np.frexp(ar[nrm])  # ar = (2 f) 2^(e2-1), 2f in [1, 2)
        e = e2 - 1
        m = np.rint((2.0 * f - 1.0) * 8.0).astype(np.int64)
        code[nrm] = ((e + 7) << 3 | m).astype(np.uint8)
    code |= np.where(np.signbit(r), 0x80, 0).astype(np.uint8)
    return code


# ------------------------------------------------------------------ int8

def int8_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 bytes -> float64 two's-complement integers (exact)."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(b >= 128, b - 256, b).astype(np.float64)


def int8_quantize_rows(w32: np.ndarray):
    """Per-row absmax scaling to symmetric int8, as the stored int8 models are built:
    s = max|w|/127 (1 for an all-zero row) in binary32, q = round-half-even(fl32(w / s))
    clamped to [-127, 127].  Returns (codes as uint8 bytes, s).

    Used only to check that the stored int8 models are what their recipe says."""
    w32 = np.asarray(w32, dtype=np.float32)
    amax = np.max(np.abs(w32), axis=1)
    s = np.where(amax > 0, (amax.astype(np.float64) / 127.0).astype(np.float32),
                 np.float32(1.0)).astype(np.float32)
    ratio = (w32.astype(np.float64) / s[:, None].astype(np.float64)).astype(np.float32)
    q = np.clip(np.rint(ratio.astype(np.float64)), -127, 127).astype(np.int64)
    return (q & 0xFF).astype(np.uint8), s


# ------------------------------------------------------------------ dispatch

def decode(codes: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "bf16":
        return bf16_decode(codes)
    if fmt == "fp8":
        return e4m3_decode(codes)
    if fmt == "int8":
        return int8_decode(codes)
    if fmt == "f64":
        return np.asarray(codes, dtype=np.float64)
    raise ValueError(fmt)


def encode(x: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "bf16":
        return bf16_encode(x)
    if fmt == "fp8":
        return e4m3_encode(x)
    if fmt == "f64":
        return np.asarray(x, dtype=np.float64).copy()
    raise ValueError(fmt)


def fp8_quantize_rows(w32: np.ndarray):
    """Per-row absmax scaling to E4M3, as the stored models are built: s = max|w|/448
    (1 for an all-zero row) in binary32, q = RNE_e4m3(fl32(w / s)).  Returns (codes, s).

    Used only to check that the stored fp8 models are what their recipe says."""
    w32 = np.asarray(w32, dtype=np.float32)
    amax = np.max(np.abs(w32), axis=1)
    s = np.where(amax > 0, (amax.astype(np.float64) / 448.0).astype(np.float32),
                 np.float32(1.0)).astype(np.float32)
    ratio = (w32.astype(np.float64) / s[:, None].astype(np.float64)).astype(np.float32)
    return e4m3_encode(ratio.astype(np.float64)), s
