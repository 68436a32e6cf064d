"""FP8 E4M3 codec, per-tensor and per-row quantisers and bfloat16 rounding
(oracle).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

Format (kongchang.com page, FP8 explainer under "Triton Backend Routing": E4M3
has a 4-bit exponent and a 3-bit mantissa).  The pages name no variant; the
one used is the OCP "fn" variant, the FP8 type of the MI355X matrix cores:

    bit 7 sign s, bits 6..3 exponent e (bias 7), bits 2..0 mantissa m
    e == 0              value = (-1)^s * m * 2^-9          (subnormals, +-0)
    1 <= e <= 15        value = (-1)^s * (1 + m/8) * 2^(e-7)
    e == 15 and m == 7  NaN (0x7F, 0xFF); there is no infinity
    largest finite      448 (0x7E)

Encoding is round-to-nearest, ties to the even mantissa, saturating to
+-448, keeping the sign of the input (so tiny negative inputs give 0x80).
The per-tensor scale is s = amax / 448 (one float32 division), with s = 1 when
amax == 0, and the codes are encode(v / s) with v / s a float32 division.
"""

import numpy as np

E4M3_MAX = 448.0

# Exponent range of the finite normal numbers and the subnormal quantum.
_EMIN = -6          # 2^-6 is the smallest normal
_MBITS = 3


def decode_table():
    """Value of each of the 256 codes (float64; NaN for 0x7F and 0xFF)."""
    codes = np.arange(256, dtype=np.int64)
    s = (codes >> 7) & 1
    e = (codes >> 3) & 0xF
    m = codes & 0x7
    mag = np.where(e == 0,
                   m * 2.0 ** (_EMIN - _MBITS),
                   (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where(s == 1, -mag, mag)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return val


def decode(codes):
    """Float64 values of uint8 codes."""
    return decode_table()[np.asarray(codes, dtype=np.uint8)]


def encode(v):
    """E4M3 codes (uint8) of float values, RNE with saturation to +-448.

    Works in float64, where every step below is exact for float32 or float64
    inputs of finite value: dividing by a power of two, ``np.rint`` (round
    half to even) and multiplying back.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN has no saturating E4M3 encoding here")
    sign = np.signbit(v)
    a = np.abs(v)
    # floor(log2(a)) exactly, via frexp: a = f * 2^x with f in [0.5, 1).
    _, x = np.frexp(np.where(a > 0, a, 1.0))
    flog = np.maximum(x - 1, _EMIN)                 # binade of the quantum
    quantum = np.exp2((flog - _MBITS).astype(np.float64))
    r = np.rint(a / quantum) * quantum              # nearest, ties to even
    r = np.minimum(r, E4M3_MAX)                     # saturate (also inf)
    # bits of the (now representable) magnitude r
    _, xr = np.frexp(np.where(r > 0, r, 1.0))
    er = xr - 1
    sub = (r < 2.0 ** _EMIN)
    exp_field = np.where(sub, 0, er + 7)
    mant = np.where(sub,
                    r / 2.0 ** (_EMIN - _MBITS),
                    (r / np.exp2(er.astype(np.float64)) - 1.0) * 8.0)
    mant = np.rint(mant).astype(np.int64)
    exp_field = np.where(r == 0, 0, exp_field).astype(np.int64)
    code = (exp_field << 3) | mant
    code = np.where(sign, code | 0x80, code)
    return code.astype(np.uint8)


def per_tensor_scale(v):
    """s = amax|v| / 448 as one float32 division; 1 when amax is 0."""
    v = np.asarray(v, dtype=np.float32)
    amax = np.float32(np.max(np.abs(v))) if v.size else np.float32(0.0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(E4M3_MAX))


def quantize(v, scale=None):
    """(codes, scale) of the per-tensor E4M3 quantisation of float32 values.

    ``v`` is first rounded to float32 (the device holds it there); the scale is
    ``per_tensor_scale(v)`` unless given; each code is encode(v / s) with the
    quotient rounded to float32, as an IEEE float32 division gives it.
    """
    v32 = np.asarray(v, dtype=np.float32)
    s = per_tensor_scale(v32) if scale is None else np.float32(scale)
    q = (v32 / s).astype(np.float32)
    return encode(q), s


def quantize_rows(v):
    """(codes, scales) of the E4M3 quantisation of each row with its own scale.

    Finer granularity, read from the kongchang.com page, "Triton Backend
    Routing: A Practical Path to FP8 Quantization" (numerical distributions
    differ, so one uniform scale loses precision; here carried from experts
    down to weight channels and activation rows): row r gets
    s_r = amax|v_r| / 448 (``per_tensor_scale`` of the row alone) and codes
    encode(v_r / s_r).  ``v`` is [R, C]; returns codes [R, C] uint8 and scales
    [R] float32.
    """
    v32 = np.asarray(v, dtype=np.float32)
    if v32.ndim != 2:
        raise ValueError("quantize_rows expects a 2-D array")
    codes = np.empty(v32.shape, dtype=np.uint8)
    scales = np.empty(v32.shape[0], dtype=np.float32)
    for r in range(v32.shape[0]):
        codes[r], scales[r] = quantize(v32[r])
    return codes, scales


def dequantize(codes, scale):
    """code value * scale in float64."""
    return decode(codes) * np.float64(scale)


# --------------------------------------------------------------------------
# bfloat16
# --------------------------------------------------------------------------

def bf16_round(v):
    """Round float32 values to bfloat16, nearest-even; returned as float32.

    bfloat16 is the upper half of a float32.  Adding 0x7FFF plus the lowest
    kept bit to the bit pattern and truncating is round-to-nearest-even for
    finite values.  NaN is not expected here.
    """
    v = np.asarray(v, dtype=np.float32)
    bits = v.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32).reshape(v.shape)


def bf16_bits(v):
    """bfloat16 bit patterns (uint16) of float32 values, nearest-even."""
    return (bf16_round(v).view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(bits):
    """float32 values of bfloat16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)
