"""Storage encodings used by the latent cache — oracle side (TEST INFRASTRUCTURE ONLY).

The attention reads the *stored* cache row, so the oracle rounds every row it appends exactly
the way storage does, with its own code (no GPU code, no shared tables):

* bf16: round-to-nearest-even from float32 (bit-level, written here).
* fp16: IEEE binary16 round-to-nearest-even (numpy's float16 cast, a library primitive).
* fp8 e4m3 (OCP "e4m3fn": bias 7, largest finite 448, no infinities, 0x7F/0xFF = NaN) with one
  float32 scale per token: scale = amax / 448 (1 when the row is all zero), code = RNE(x / scale)
  saturated to +-448, dequantised value = code * scale.

* fp6 e2m3 (OCP MX "FP6 E2M3": sign, 2 exponent bits with bias 1, 3 mantissa bits, subnormals
  m/8, largest finite 7.5, no infinities and no NaN) with one float32 scale per token:
  scale = amax / 7.5 (1 when the row is all zero), code = RNE(x / scale) saturated to +-7.5 (a NaN
  input encodes as +0: the format has no NaN), dequantised value = code * scale. A row of n codes
  is stored as a little-endian bit stream of n * 6 bits: code j occupies bits 6j .. 6j + 5, bit b
  of the stream being bit (b mod 8) of byte b / 8.

The pages give no low-bit format: the review page says only that the deployed cache averages
about six bits per element (section 4.2 "Evaluation", inference efficiency) and the summary page
repeats "6-bit" for the 8xH800 deployment. The e4m3 and e2m3 per-token-scale formats above are
readings made for this library, not the pages' format (e2m3 + a 4-byte scale is 6.06 bits per
element at 576 elements per row). The scale division and the encoding decision are taken in
float32, the precision the GPU kernels take them in.

Pins: tests/test_encodings.py (all 256 e4m3 codes against torch's float8_e4m3fn, RNE ties,
saturation, bf16 against torch's bfloat16 cast on every 16-bit pattern class, fp16 against torch;
all 64 e2m3 codes against the format's definition written out by hand, the e2m3 encoder against a
brute-force nearest-value search with ties to even, the packed bit positions).
"""
import numpy as np

_F32 = np.float32


def bf16_encode(x) -> np.ndarray:
    """float -> bf16 bit pattern (uint16), RNE from float32. Input is first rounded to float32."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(_F32))
    u = x32.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x32)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    r = np.where(nan, 0x7FC0, r)
    return r.astype(np.uint16)


def bf16_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint16).astype(np.uint32) << 16
    return np.ascontiguousarray(c).view(_F32).astype(np.float64)


def fp16_encode(x) -> np.ndarray:
    x32 = np.asarray(x, dtype=np.float64).astype(_F32)
    with np.errstate(over="ignore"):
        return x32.astype(np.float16).view(np.uint16)


def fp16_decode(codes) -> np.ndarray:
    return np.asarray(codes, dtype=np.uint16).view(np.float16).astype(np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """e4m3 code -> value (float64), following the format's definition bit by bit."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * (1.0 + m / 8.0) * np.power(2.0, e - 7)
    sub = sign * (m / 8.0) * 2.0 ** (-6)
    v = np.where(e == 0, sub, normal)
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return v


def e4m3_encode(x32) -> np.ndarray:
    """float32 value -> e4m3 code, round-to-nearest-even, saturating at +-448, NaN -> 0x7F.

    Works on the exact binary value of the float32 input: the magnitude is written as an integer
    multiple q of the target spacing (2^-9 below 2^-6, else 2^(E-3) in binade [2^E, 2^(E+1)))
    plus a remainder in [0, 1); the remainder decides the rounding (ties to even q)."""
    x = np.asarray(x32, dtype=_F32).astype(np.float64)   # exact widening
    nan = np.isnan(x)
    x = np.where(nan, 0.0, np.clip(x, -896.0, 896.0))    # beyond 448 everything saturates
    neg = np.signbit(x)
    a = np.abs(x)
    _, E = np.frexp(a)                 # a = m * 2^E with 0.5 <= m < 1 (E = 0 for a = 0)
    E = E.astype(np.int64) - 1         # a in [2^E, 2^(E+1))
    qexp = np.where(E < -6, -9, E - 3)
    scaled = np.ldexp(a, -qexp)        # exact: power-of-two scaling
    q = np.floor(scaled)
    frac = scaled - q
    q = q + ((frac > 0.5) | ((frac == 0.5) & (np.fmod(q, 2.0) == 1.0)))
    val = np.minimum(np.ldexp(q, qexp), 448.0)
    # field encoding of the rounded magnitude
    sub = val < 2.0 ** -6
    _, E2 = np.frexp(np.where(sub, 1.0, val))
    E2 = E2.astype(np.int64) - 1
    mant_norm = np.rint((np.ldexp(np.where(sub, 1.0, val), -E2) - 1.0) * 8.0).astype(np.int64)
    mant_sub = np.rint(np.ldexp(val, 9)).astype(np.int64)
    code = np.where(sub, mant_sub, ((E2 + 7) << 3) | mant_norm)
    code = code | np.where(neg, 0x80, 0)
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


def quantize_rows_e4m3(rows32):
    """Cache rows (float32 values, [..., row]) -> (codes uint8 [..., row], scales float32 [...]).
    Per row: scale = amax / 448 in float32 (1 for an all-zero row); code = e4m3(x / scale)."""
    r = np.asarray(rows32, dtype=_F32)
    amax = np.max(np.abs(r), axis=-1).astype(_F32)
    scale = np.where(amax == 0, _F32(1.0), (amax / _F32(448.0)).astype(_F32)).astype(_F32)
    q = (r / scale[..., None]).astype(_F32)    # float32 division, correctly rounded
    return e4m3_encode(q), scale


def quantize_row_e4m3(row32):
    """One cache row -> (codes, scale)."""
    codes, scale = quantize_rows_e4m3(np.asarray(row32, dtype=_F32)[None, :])
    return codes[0], _F32(scale[0])


def e2m3_decode(codes) -> np.ndarray:
    """e2m3 code (low 6 bits) -> value (float64), following the format's definition bit by bit."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64) & 0x3F
    sign = np.where(c & 0x20, -1.0, 1.0)
    e = (c >> 3) & 0x3
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.power(2.0, e - 1)
    sub = m / 8.0
    return sign * np.where(e == 0, sub, normal)


def e2m3_encode(x32) -> np.ndarray:
    """float32 value -> e2m3 code (uint8 holding 6 bits), round-to-nearest-even on the exact binary
    value, saturating at +-7.5; NaN -> +0.

    The magnitude is written as an integer multiple q of the format's spacing at that magnitude
    (1/8 below 1, else 2^(E-3) in binade [2^E, 2^(E+1))) plus a remainder in [0, 1), which decides
    the rounding (ties to even q)."""
    x = np.asarray(x32, dtype=_F32).astype(np.float64)   # exact widening
    nan = np.isnan(x)
    x = np.where(nan, 0.0, np.clip(x, -16.0, 16.0))      # beyond 7.5 everything saturates
    neg = np.signbit(x) & ~nan
    a = np.abs(x)
    _, E = np.frexp(a)
    E = E.astype(np.int64) - 1                           # a in [2^E, 2^(E+1)) (a > 0)
    qexp = np.where(E < 0, -3, E - 3)
    scaled = np.ldexp(a, -qexp)
    q = np.floor(scaled)
    frac = scaled - q
    q = q + ((frac > 0.5) | ((frac == 0.5) & (np.fmod(q, 2.0) == 1.0)))
    val = np.minimum(np.ldexp(q, qexp), 7.5)
    sub = val < 1.0
    _, E2 = np.frexp(np.where(sub, 1.0, val))
    E2 = E2.astype(np.int64) - 1
    mant_norm = np.rint((np.ldexp(np.where(sub, 1.0, val), -E2) - 1.0) * 8.0).astype(np.int64)
    mant_sub = np.rint(val * 8.0).astype(np.int64)
    code = np.where(sub, mant_sub, ((E2 + 1) << 3) | mant_norm)
    code = code | np.where(neg, 0x20, 0)
    return code.astype(np.uint8)


def pack_e2m3(codes) -> np.ndarray:
    """[..., n] 6-bit codes -> [..., n * 6 / 8] bytes, little-endian bit stream (n a multiple of 4)."""
    c = np.asarray(codes, dtype=np.uint8)
    n = c.shape[-1]
    assert n % 4 == 0
    bits = ((c[..., :, None].astype(np.uint16) >> np.arange(6, dtype=np.uint16)) & 1).astype(np.uint8)
    bits = bits.reshape(c.shape[:-1] + (n * 6 // 8, 8))          # bit b of the stream at [b // 8, b % 8]
    return (bits.astype(np.uint16) << np.arange(8, dtype=np.uint16)).sum(-1).astype(np.uint8)


def unpack_e2m3(packed, n) -> np.ndarray:
    """Inverse of pack_e2m3: [..., n * 6 / 8] bytes -> [..., n] codes."""
    p = np.asarray(packed, dtype=np.uint8)
    bits = ((p[..., :, None].astype(np.uint16) >> np.arange(8, dtype=np.uint16)) & 1).astype(np.uint8)
    bits = bits.reshape(p.shape[:-1] + (n, 6))
    return (bits.astype(np.uint16) << np.arange(6, dtype=np.uint16)).sum(-1).astype(np.uint8)


def quantize_rows_e2m3(rows32):
    """Cache rows (float32 values, [..., row]) -> (codes uint8 [..., row], scales float32 [...]).
    Per row: scale = amax / 7.5 in float32 (1 for an all-zero row); code = e2m3(x / scale)."""
    r = np.asarray(rows32, dtype=_F32)
    amax = np.max(np.abs(r), axis=-1).astype(_F32)
    scale = np.where(amax == 0, _F32(1.0), (amax / _F32(7.5)).astype(_F32)).astype(_F32)
    q = (r / scale[..., None]).astype(_F32)    # float32 division, correctly rounded
    return e2m3_encode(q), scale


def store_rows(rows, cdtype):
    """Round rows (float64/float32, [..., row]) to storage. Returns (payload, scales-or-None)."""
    rows = np.asarray(rows)
    if cdtype == "f32":
        return rows.astype(_F32), None
    if cdtype == "bf16":
        return bf16_encode(rows), None
    if cdtype == "f16":
        return fp16_encode(rows), None
    if cdtype == "fp8_e4m3":
        return quantize_rows_e4m3(rows.astype(_F32))
    if cdtype == "fp6_e2m3":
        codes, scales = quantize_rows_e2m3(rows.astype(_F32))
        return pack_e2m3(codes), scales
    raise ValueError(cdtype)


def load_rows(payload, cdtype, scales=None) -> np.ndarray:
    """Stored rows -> float64 values the attention sees."""
    if cdtype == "f32":
        return np.asarray(payload, dtype=_F32).astype(np.float64)
    if cdtype == "bf16":
        return bf16_decode(payload)
    if cdtype == "f16":
        return fp16_decode(payload)
    if cdtype == "fp8_e4m3":
        v = e4m3_decode(payload)
        return v * np.asarray(scales, dtype=_F32).astype(np.float64)[..., None]
    if cdtype == "fp6_e2m3":
        p = np.asarray(payload, dtype=np.uint8)
        v = e2m3_decode(unpack_e2m3(p, p.shape[-1] * 8 // 6))
        return v * np.asarray(scales, dtype=_F32).astype(np.float64)[..., None]
    raise ValueError(cdtype)
