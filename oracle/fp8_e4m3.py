"""OCP 8-bit floating point, E4M3 ("e4m3fn") codec for the oracle.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Format (OCP 8-bit Floating Point Specification, E4M3): 1 sign, 4 exponent
bits with bias 7, 3 mantissa bits; subnormals when the exponent field is 0
(value m * 2^-9); no infinities; S.1111.111 is NaN; largest finite 448.

Block quantisation as the DeepSeek-deployment page states it (Quantization
section): activations get one scale per 128-element vector, weights one per
128x128 block.  The pages give only the granularity; the constants here are
the plainest reading: scale = amax / 448 in fp32, scale = 1 for an all-zero
group, code = round-to-nearest-even of clamp(v / scale, -448, 448).
"""
import numpy as np

E4M3_MAX = np.float32(448.0)


def _decode_fields(c: np.ndarray) -> np.ndarray:
    """Value of each e4m3fn code, from its sign / exponent / mantissa fields."""
    c = c.astype(np.int32)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = c & 0x7
    mag = np.where(ef == 0, mf * 2.0 ** -9, (1.0 + mf / 8.0) * np.exp2(ef - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return (sign * mag).astype(np.float32)


_TABLE = _decode_fields(np.arange(256))


def e4m3_table() -> np.ndarray:
    """The 256 decoded values, indexed by code."""
    return _TABLE.copy()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each e4m3fn code (a lookup in the 256-entry table of field values)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even encoding of finite fp32 values, saturating at +-448."""
    v = np.asarray(v, dtype=np.float32)
    assert np.all(np.isfinite(v)), "e4m3_encode: non-finite input"
    a = np.minimum(np.abs(v).astype(np.float64), 448.0)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int32)
    # Subnormal range |v| < 2^-6: the value is m * 2^-9 with m in 0..8
    # (m == 8 is the smallest normal, code 0x08).  a * 2^9 is exact.
    m_sub = np.rint(a * 2.0 ** 9).astype(np.int32)           # rint: half to even
    # Normal range: a = f * 2^ex with f in [0.5, 1), so a = (2f) * 2^(ex-1).
    f, ex = np.frexp(np.where(a > 0, a, 1.0))
    e_unb = ex - 1
    mant = np.rint((2.0 * f - 1.0) * 8.0).astype(np.int32)   # exact scaling, half to even
    carry = mant == 8
    e_unb = np.where(carry, e_unb + 1, e_unb)
    mant = np.where(carry, 0, mant)
    code_norm = ((e_unb + 7) << 3) | mant
    code = np.where(a < 2.0 ** -6, m_sub, code_norm)
    return (sign | code).astype(np.uint8)


def quantize_groups_128(v: np.ndarray):
    """Per-row, per-128-column-group quantisation of an fp32 [rows, C] matrix.

    Returns (codes uint8 [rows, C], scales fp32 [rows, C/128]).
    """
    v = np.asarray(v, dtype=np.float32)
    rows, C = v.shape
    assert C % 128 == 0
    g = v.reshape(rows, C // 128, 128)
    amax = np.abs(g).max(axis=-1)
    scale = np.where(amax == 0, np.float32(1.0), amax / E4M3_MAX).astype(np.float32)
    q = np.clip(g / scale[..., None], -E4M3_MAX, E4M3_MAX).astype(np.float32)
    return e4m3_encode(q).reshape(rows, C), scale


def dequantize_groups_128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    rows, C = codes.shape
    vals = e4m3_decode(codes).reshape(rows, C // 128, 128)
    return (vals * scales[..., None]).reshape(rows, C).astype(np.float32)


def dequantize_blocks_128x128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Weight matrix [N, K] from codes and one scale per 128x128 block [N/128, K/128]."""
    n, k = codes.shape
    vals = e4m3_decode(codes).reshape(n // 128, 128, k // 128, 128)
    return (vals * scales[:, None, :, None]).reshape(n, k).astype(np.float32)
