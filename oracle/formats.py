"""Element formats of the oracle: 16-bit floats and OCP e4m3fn, to/from fp64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

e4m3fn is written out from its definition (OCP 8-bit floating point, the
format behind the "FP8 KV Cache" feature named on the ChunkLlama/vLLM feature
list page): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent
field 0 holds subnormals m * 2**-9; there are no infinities; S.1111.111 is NaN;
the largest finite magnitude is 1.75 * 2**8 = 448.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


def f16_to_f64(a: np.ndarray) -> np.ndarray:
    """IEEE binary16 values -> fp64 (exact)."""
    assert a.dtype == np.float16
    return a.astype(np.float64)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> fp64 (exact): a bfloat16 is the upper
    half of a binary32 with the same sign and exponent."""
    assert bits.dtype == np.uint16
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """e4m3fn codes (uint8) -> fp64, field by field from the definition."""
    assert codes.dtype == np.uint8
    c = codes.astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    out[(e == 0xF) & ((c & 0x7) == 0x7)] = np.nan
    return out


def to_f64(a: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "f16":
        return f16_to_f64(a)
    if fmt == "bf16":
        return bf16_to_f64(a)
    if fmt == "e4m3fn":
        return e4m3fn_to_f64(a)
    if fmt in ("f32", "f64"):
        return np.asarray(a, dtype=np.float64)
    raise ValueError(f"unknown element format {fmt!r}")


def _e4m3fn_code_of_value(v: float) -> int:
    """Code of an exactly representable finite e4m3fn value."""
    s = 0x80 if (v < 0 or (v == 0 and math.copysign(1.0, v) < 0)) else 0
    a = abs(v)
    if a < 2.0 ** -6:                       # subnormal (or zero): a = m * 2**-9
        m = a / 2.0 ** -9
        assert m == int(m) and 0 <= m <= 7
        return s | int(m)
    e = math.floor(math.log2(a))
    frac = a / 2.0 ** e - 1.0               # in [0, 1), multiple of 1/8
    m = frac * 8.0
    assert m == int(m) and 0 <= m <= 7 and -6 <= e <= 8
    return s | ((e + 7) << 3) | int(m)


def e4m3fn_round(y: float) -> float:
    """Round one binary32 value to e4m3fn: clamp to [-448, 448], then round to
    the nearest representable value, ties to the value with an even mantissa
    field.  NaN stays NaN."""
    if y != y:
        return y
    y = max(-E4M3_MAX, min(E4M3_MAX, y))
    a = abs(y)
    # quantum of the binade that holds a (subnormal binade shares 2**-9)
    e = max(math.floor(math.log2(a)), -6) if a > 0 else -6
    quantum = 2.0 ** (e - 3)
    n = a / quantum                          # exact: a is binary32, quantum a power of 2
    lo = math.floor(n)
    rem = n - lo
    if rem > 0.5 or (rem == 0.5 and lo % 2 == 1):
        lo += 1
    return math.copysign(lo * quantum, y)


def e4m3fn_encode(x: np.ndarray, inv_scale: np.float32) -> np.ndarray:
    """Quantise: code = e4m3fn(clamp(fp32(x) * fp32(inv_scale), +-448)).

    The product is a binary32 multiply (this decides the code, so it is taken
    in the precision the cache writer uses); the rounding to e4m3fn is exact
    arithmetic.  NaN inputs give the NaN code with the input's sign (0x7F or
    0xFF)."""
    with np.errstate(invalid="ignore", over="ignore"):
        y = (np.asarray(x, dtype=np.float32) * np.float32(inv_scale)).astype(np.float32)
    flat = y.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for i, val in enumerate(flat.tolist()):
        if val != val:
            out[i] = 0xFF if math.copysign(1.0, val) < 0 else 0x7F
            continue
        out[i] = _e4m3fn_code_of_value(e4m3fn_round(val))
    return out.reshape(y.shape)


def inv_scale_f32(scale: float) -> np.float32:
    """1/scale as one binary32 division (the cache writer's quantiser factor)."""
    return np.float32(np.float32(1.0) / np.float32(scale))


def quantise_e4m3fn(x: np.ndarray, scale: float) -> np.ndarray:
    """Codes an e4m3fn cache with per-tensor scale `scale` stores for the
    values x (value = code * scale): the binary32 reciprocal of the scale is
    taken once, each binary32 x is multiplied by it in binary32, and the
    product is clamped and rounded to e4m3fn (e4m3fn_encode)."""
    return e4m3fn_encode(np.asarray(x, dtype=np.float32), inv_scale_f32(scale))
