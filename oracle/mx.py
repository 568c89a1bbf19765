"""Microscaling (MX) FP8 quantisation, E4M3 elements, for the oracle.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages name the format and its block: "Hosting Qwen on Blackwell"
(Quantization) serves Qwen3-235B with MXFP8 weights converted statically,
and "CuTeDSL at Perplexity" (closing section on Blackwell's quantisation
schemes) computes the absolute maximum over 32 elements for MXFP8.  They do
not spell out the scale; the plainest reading is the OCP Microscaling (MX)
v1.0 definition of MXFP8 (E4M3):
  - a block is 32 consecutive values along the contraction dimension;
  - its shared scale is the power of two X = 2^(floor(log2(amax)) - 8), 8
    being the exponent of E4M3's largest normal (448 = 1.75 * 2^8), stored as
    an E8M0 code (exponent + 127);
  - each element is the E4M3 code of v / X, rounded to nearest even and
    saturated at +-448 (|v / X| < 512, so only the top of the range clips).
Where that definition leaves a choice, this oracle takes: an all-zero block
gets the smallest scale 2^-127 (code 0) and zero elements; exponents are
clamped to [-127, 127].
"""
import numpy as np

from .fp8_e4m3 import e4m3_decode, e4m3_encode

MX_BLOCK = 32
E4M3_EMAX = 8


def mx_scale_exponent(amax: np.ndarray) -> np.ndarray:
    """floor(log2(amax)) - 8 per block, clamped to [-127, 127]; -127 for amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    # amax = f * 2^ex with f in [0.5, 1): floor(log2(amax)) = ex - 1 (exact).
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    e = np.where(amax > 0, ex - 1 - E4M3_EMAX, -127)
    return np.clip(e, -127, 127).astype(np.int32)


def mx_quantize_rows(v: np.ndarray):
    """MXFP8 of an fp32 [rows, C] matrix, blocks of 32 along each row.

    Returns (codes uint8 [rows, C], e8m0 uint8 [rows, C/32]).
    """
    v = np.asarray(v, dtype=np.float32)
    rows, C = v.shape
    assert C % MX_BLOCK == 0
    g = v.reshape(rows, C // MX_BLOCK, MX_BLOCK).astype(np.float64)
    e = mx_scale_exponent(np.abs(g).max(axis=-1))
    q = g * np.exp2(-e.astype(np.float64))[..., None]      # exact: a power-of-two scaling
    codes = e4m3_encode(q.astype(np.float32)).reshape(rows, C)
    return codes, (e + 127).astype(np.uint8)


def mx_dequantize_rows(codes: np.ndarray, e8m0: np.ndarray) -> np.ndarray:
    """fp32 values code * 2^(e8m0 - 127), blocks of 32 along each row (exact)."""
    rows, C = codes.shape
    vals = e4m3_decode(codes).astype(np.float64).reshape(rows, C // MX_BLOCK, MX_BLOCK)
    scale = np.exp2(e8m0.astype(np.float64) - 127.0)
    return (vals * scale[..., None]).reshape(rows, C).astype(np.float32)
