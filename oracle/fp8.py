"""FP8 codecs (E4M3 and E5M2), per-tensor and per-row quantisers and
bfloat16 rounding (oracle).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

Formats (kongchang.com page, FP8 explainer under "Triton Backend Routing":
E4M3 has a 4-bit exponent and a 3-bit mantissa, smaller range and more
precision; E5M2 a 5-bit exponent and a 2-bit mantissa, larger range and less
precision).  The pages name no variant; the ones used are the OCP formats of
the MI355X matrix cores:

  E4M3 ("fn"): bit 7 sign, bits 6..3 exponent e (bias 7), bits 2..0 mantissa m
    e == 0              value = (-1)^s * m * 2^-9          (subnormals, +-0)
    1 <= e <= 15        value = (-1)^s * (1 + m/8) * 2^(e-7)
    e == 15 and m == 7  NaN (0x7F, 0xFF); there is no infinity
    largest finite      448 (0x7E)
  E5M2: bit 7 sign, bits 6..2 exponent e (bias 15), bits 1..0 mantissa m
    e == 0              value = (-1)^s * m * 2^-16         (subnormals, +-0)
    1 <= e <= 30        value = (-1)^s * (1 + m/4) * 2^(e-15)
    e == 31             infinity (m == 0) or NaN
    largest finite      57344 (0x7B)

Encoding is round-to-nearest, ties to the even mantissa, saturating to the
largest finite value, keeping the sign of the input (so tiny negative inputs
give 0x80).  The per-tensor scale is s = amax / max (one float32 division),
with s = 1 when amax == 0, and the codes are encode(v / s) with v / s a
float32 division.
"""

import numpy as np

E4M3_MAX = 448.0
E5M2_MAX = 57344.0

# Per format: exponent bias, mantissa bits, largest finite value; the
# smallest normal is 2^(1 - bias).
FORMATS = {
    "e4m3": dict(bias=7, mbits=3, max=E4M3_MAX),
    "e5m2": dict(bias=15, mbits=2, max=E5M2_MAX),
}


def _fmt(fmt):
    if fmt not in FORMATS:
        raise ValueError(f"unknown FP8 format {fmt!r}")
    return FORMATS[fmt]


def fp8_max(fmt="e4m3"):
    return _fmt(fmt)["max"]


def decode_table(fmt="e4m3"):
    """Value of each of the 256 codes (float64; NaN / inf where the format
    has them)."""
    f = _fmt(fmt)
    bias, mb = f["bias"], f["mbits"]
    ebits = 7 - mb
    emax_field = (1 << ebits) - 1
    codes = np.arange(256, dtype=np.int64)
    s = (codes >> 7) & 1
    e = (codes >> mb) & emax_field
    m = codes & ((1 << mb) - 1)
    mag = np.where(e == 0,
                   m * 2.0 ** (1 - bias - mb),
                   (1.0 + m / float(1 << mb)) * np.exp2(e.astype(np.float64) - bias))
    if fmt == "e4m3":
        mag = np.where((e == emax_field) & (m == (1 << mb) - 1), np.nan, mag)
    else:
        mag = np.where(e == emax_field, np.where(m == 0, np.inf, np.nan), mag)
    return np.where(s == 1, -mag, mag)


def decode(codes, fmt="e4m3"):
    """Float64 values of uint8 codes."""
    return decode_table(fmt)[np.asarray(codes, dtype=np.uint8)]


def encode(v, fmt="e4m3"):
    """FP8 codes (uint8) of float values, RNE with saturation to +-max.

    Works in float64, where every step below is exact for float32 or float64
    inputs of finite value: dividing by a power of two, ``np.rint`` (round
    half to even) and multiplying back.
    """
    f = _fmt(fmt)
    bias, mb, vmax = f["bias"], f["mbits"], f["max"]
    emin = 1 - bias                                  # binade of the smallest normal
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN has no saturating FP8 encoding here")
    sign = np.signbit(v)
    a = np.abs(v)
    # floor(log2(a)) exactly, via frexp: a = f * 2^x with f in [0.5, 1).
    _, x = np.frexp(np.where(a > 0, a, 1.0))
    flog = np.maximum(x - 1, emin)                   # binade of the quantum
    quantum = np.exp2((flog - mb).astype(np.float64))
    r = np.rint(a / quantum) * quantum               # nearest, ties to even
    r = np.minimum(r, vmax)                          # saturate (also inf)
    # bits of the (now representable) magnitude r
    _, xr = np.frexp(np.where(r > 0, r, 1.0))
    er = xr - 1
    sub = (r < 2.0 ** emin)
    exp_field = np.where(sub, 0, er + bias)
    mant = np.where(sub,
                    r / 2.0 ** (emin - mb),
                    (r / np.exp2(er.astype(np.float64)) - 1.0) * float(1 << mb))
    mant = np.rint(mant).astype(np.int64)
    exp_field = np.where(r == 0, 0, exp_field).astype(np.int64)
    code = (exp_field << mb) | mant
    code = np.where(sign, code | 0x80, code)
    return code.astype(np.uint8)


def per_tensor_scale(v, fmt="e4m3"):
    """s = amax|v| / max as one float32 division; 1 when amax is 0."""
    v = np.asarray(v, dtype=np.float32)
    amax = np.float32(np.max(np.abs(v))) if v.size else np.float32(0.0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(fp8_max(fmt)))


def quantize(v, scale=None, fmt="e4m3"):
    """(codes, scale) of the per-tensor FP8 quantisation of float32 values.

    ``v`` is first rounded to float32 (the device holds it there); the scale is
    ``per_tensor_scale(v)`` unless given; each code is encode(v / s) with the
    quotient rounded to float32, as an IEEE float32 division gives it.
    """
    v32 = np.asarray(v, dtype=np.float32)
    s = per_tensor_scale(v32, fmt) if scale is None else np.float32(scale)
    q = (v32 / s).astype(np.float32)
    return encode(q, fmt), s


def quantize_rows(v, fmt="e4m3"):
    """(codes, scales) of the FP8 quantisation of each row with its own scale.

    Finer granularity, read from the kongchang.com page, "Triton Backend
    Routing: A Practical Path to FP8 Quantization" (numerical distributions
    differ, so one uniform scale loses precision; here carried from experts
    down to weight channels and activation rows): row r gets
    s_r = amax|v_r| / max (``per_tensor_scale`` of the row alone) and codes
    encode(v_r / s_r).  ``v`` is [R, C]; returns codes [R, C] uint8 and scales
    [R] float32.
    """
    v32 = np.asarray(v, dtype=np.float32)
    if v32.ndim != 2:
        raise ValueError("quantize_rows expects a 2-D array")
    codes = np.empty(v32.shape, dtype=np.uint8)
    scales = np.empty(v32.shape[0], dtype=np.float32)
    for r in range(v32.shape[0]):
        codes[r], scales[r] = quantize(v32[r], fmt=fmt)
    return codes, scales


def dequantize(codes, scale, fmt="e4m3"):
    """code value * scale in float64."""
    return decode(codes, fmt) * np.float64(scale)


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
