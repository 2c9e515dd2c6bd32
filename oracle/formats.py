"""Storage formats used by the fused matmul + collective path, written from their definitions.

Test infrastructure only (see oracle/__init__.py).

The pages fix fp16 as the w8A16 format and leave the storage and accumulation
types of the other ops open (CoC guide, "Approach - fused-kernel
implementation", last item of the fused-operator list).  The readings used here:
operands and partial sums are stored in the op's dtype (fp32, fp16 or bf16) and
every conversion from a wider value rounds to nearest, ties to even (RNE).

Both 16-bit formats are IEEE-style binary formats with 1 sign bit, an exponent
field with bias ``2**(ebits-1) - 1``, an all-ones exponent for inf/NaN, an
all-zeros exponent for zero/subnormals, and a hidden leading one for normals:

    format    exponent bits  fraction bits  precision p  emin
    binary16        5              10            11       -14
    bfloat16        8               7             8      -126

Rounding a real x to such a format: the spacing of representable values
around x is ``2**(e - p + 1)`` where ``e = floor(log2|x|)``, except below the
normal range where it stays at ``2**(emin - p + 1)``.  x / spacing is rounded
to the nearest integer, halfway cases to the even one, and results above the
largest finite value overflow to infinity.
"""
from __future__ import annotations

import numpy as np

# name: (exponent bits, fraction bits)
_FORMATS = {
    "f16": (5, 10),
    "bf16": (8, 7),
}


def _params(fmt: str):
    ebits, fbits = _FORMATS[fmt]
    bias = (1 << (ebits - 1)) - 1
    p = fbits + 1                      # precision incl. hidden bit
    emin = 1 - bias                    # smallest normal exponent
    emax = bias                        # largest finite exponent
    max_finite = (2.0 - 2.0 ** (-fbits)) * 2.0 ** emax
    return ebits, fbits, bias, p, emin, emax, max_finite


def round_to(x, fmt: str) -> np.ndarray:
    """Round float64 values to the nearest value of ``fmt`` (ties to even).

    Returns float64 values that are exactly representable in ``fmt``; overflow
    gives +-inf, NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    _, _, _, p, emin, _, max_finite = _params(fmt)
    out = np.array(x, dtype=np.float64, copy=True)
    finite = np.isfinite(x) & (x != 0.0)
    if np.any(finite):
        xf = x[finite]
        # frexp: xf = f * 2**E with 0.5 <= |f| < 1, so floor(log2|xf|) = E - 1.
        _, E = np.frexp(xf)
        e = E.astype(np.int64) - 1
        spacing_exp = np.maximum(e, emin) - (p - 1)
        scaled = np.ldexp(xf, -spacing_exp)          # exact: power-of-two scaling
        q = np.rint(scaled)                           # round half to even
        r = np.ldexp(q, spacing_exp)
        r = np.where(np.abs(r) > max_finite, np.copysign(np.inf, xf), r)
        out[finite] = r
    return out


def encode(x, fmt: str) -> np.ndarray:
    """Bit pattern (uint16) of ``round_to(x, fmt)``."""
    ebits, fbits, bias, p, emin, _, _ = _params(fmt)
    r = round_to(x, fmt)
    sign = np.signbit(r).astype(np.uint32) << 15
    a = np.abs(r)
    bits = np.zeros(r.shape, dtype=np.uint32)
    exp_all_ones = (1 << ebits) - 1
    isnan = np.isnan(r)
    isinf = np.isinf(r)
    bits[isinf] = exp_all_ones << fbits
    bits[isnan] = (exp_all_ones << fbits) | (1 << (fbits - 1))   # quiet NaN
    reg = np.isfinite(r) & (a != 0.0)
    if np.any(reg):
        ar = a[reg]
        _, E = np.frexp(ar)
        e = E.astype(np.int64) - 1
        sub = e < emin
        field = np.zeros(ar.shape, dtype=np.uint32)
        # subnormal: value = frac * 2**(emin - p + 1), exponent field 0
        field[sub] = np.ldexp(ar[sub], -(emin - (p - 1))).astype(np.uint32)
        # normal: value = (2**fbits + frac) * 2**(e - fbits), field e + bias
        nrm = ~sub
        frac_nrm = np.ldexp(ar[nrm], -(e[nrm] - fbits)) - float(1 << fbits)
        field[nrm] = ((e[nrm] + bias).astype(np.uint32) << fbits) | frac_nrm.astype(np.uint32)
        bits[reg] = field
    return (bits | sign).astype(np.uint16)


def decode(bits, fmt: str) -> np.ndarray:
    """float64 value of uint16 bit patterns in ``fmt``."""
    ebits, fbits, bias, p, emin, _, _ = _params(fmt)
    b = np.asarray(bits).astype(np.uint32)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    ef = (b >> fbits) & ((1 << ebits) - 1)
    fr = (b & ((1 << fbits) - 1)).astype(np.float64)
    exp_all_ones = (1 << ebits) - 1
    val = np.where(
        ef == 0,
        np.ldexp(fr, emin - (p - 1)),
        np.ldexp(fr + float(1 << fbits), ef.astype(np.int64) - bias - fbits),
    )
    val = np.where(ef == exp_all_ones, np.where(fr == 0, np.inf, np.nan), val)
    return sign * val


def round_f32(x) -> np.ndarray:
    """Nearest binary32 value (ties to even), as float64.

    numpy's float64 -> float32 cast is the IEEE conversion, so it serves as
    this step directly.
    """
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_dtype(x, dtype: str) -> np.ndarray:
    """Round to the storage dtype of an op: 'f32', 'f16' or 'bf16'."""
    if dtype == "f32":
        return round_f32(x)
    return round_to(x, dtype)


def decode_dtype(raw, dtype: str) -> np.ndarray:
    """float64 values of raw storage: float32 array for 'f32', uint16 bits otherwise."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    return decode(np.asarray(raw).view(np.uint16), dtype)
