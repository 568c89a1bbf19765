"""Pins of the oracle's MXFP8 codec (oracle/mx.py) against what the format
fixes: closed-form scale exponents, an exhaustive nearest-code search over
the 256 E4M3 codes, exact round trips, error bounds, and an independent
torch-based conversion.  MX blocks: "Hosting Qwen on Blackwell"
(Quantization: MXFP8 weights) and "CuTeDSL at Perplexity" (absolute maximum
over 32 elements for MXFP8); constants: the OCP Microscaling v1.0 reading
stated in oracle/mx.py."""
import numpy as np
import pytest
import torch

from oracle import e4m3_table
from oracle.mx import mx_dequantize_rows, mx_quantize_rows, mx_scale_exponent
from synth.generate import _mx_rows

TABLE = e4m3_table().astype(np.float64)
FINITE = np.isfinite(TABLE)


@pytest.mark.parametrize("amax,e", [(448.0, 0), (256.0, 0), (255.999, -1), (1.0, -8),
                                    (1.5, -8), (2.0 ** -20, -28), (3.0 * 2 ** 100, 93),
                                    (0.0, -127), (2.0 ** -130, -127), (2.0 ** -118, -126),
                                    (2.0 ** -119, -127)])
def test_scale_exponent_closed_form(amax, e):
    # floor(log2(amax)) - 8, clamped to [-127, 127]; an all-zero block -> -127
    assert int(mx_scale_exponent(np.array([amax]))[0]) == e


def _nearest_code(y):
    """RNE nearest finite E4M3 code of y, saturating at +-448 (brute force)."""
    y = float(np.clip(y, -448.0, 448.0))
    d = np.where(FINITE, np.abs(TABLE - y), np.inf)
    best = np.flatnonzero(d == d.min())
    if len(best) > 1:                                   # exact tie: even mantissa
        even = [c for c in best if (c & 1) == 0 and (TABLE[c] != 0 or np.signbit(y) == bool(c & 0x80))]
        best = even or list(best)
    c = int(best[0])
    if TABLE[c] == 0:                                   # zero keeps the sign of y
        c = 0x80 if np.signbit(y) else 0x00
    return c


def test_codes_are_the_nearest_e4m3_of_the_scaled_block():
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal((6, 64)) * 10 ** rng.uniform(-6, 6, (6, 1)),
                        rng.uniform(-1, 1, (2, 64)) * 2.0 ** 40]).astype(np.float32)
    v[0, 3] = 0.0
    v[1, :32] = 0.0                                      # an all-zero block
    codes, e8 = mx_quantize_rows(v)
    for r in range(v.shape[0]):
        for b in range(v.shape[1] // 32):
            blk = v[r, 32 * b:32 * b + 32].astype(np.float64)
            amax = np.abs(blk).max()
            e = int(np.floor(np.log2(amax))) - 8 if amax > 0 else -127
            assert int(e8[r, b]) == e + 127
            for i in range(32):
                want = _nearest_code(blk[i] / 2.0 ** e)
                got = int(codes[r, 32 * b + i])
                assert got == want or (TABLE[got] == 0 and TABLE[want] == 0), (r, b, i)


def test_largest_element_keeps_top_binade():
    # |amax / X| lies in [256, 512): its code decodes to a value in [256, 448]
    rng = np.random.default_rng(8)
    v = rng.standard_normal((16, 256)).astype(np.float32)
    codes, e8 = mx_quantize_rows(v)
    vals = TABLE[codes].reshape(16, 8, 32)
    top = np.abs(vals).max(axis=-1)
    assert np.all((top >= 256) & (top <= 448))


def test_round_trip_is_exact_on_representable_blocks():
    rng = np.random.default_rng(9)
    finite = np.flatnonzero(FINITE)
    codes = rng.choice(finite, size=(8, 64)).astype(np.uint8)
    codes[:, ::32] = 0x7C                               # 384: every block max in [256, 448]
    e8 = rng.integers(100, 150, size=(8, 2)).astype(np.uint8)
    v = mx_dequantize_rows(codes, e8)
    c2, e2 = mx_quantize_rows(v)
    assert np.array_equal(e2, e8)
    assert np.array_equal(TABLE[c2], TABLE[codes])      # +0 / -0 may differ in code


def test_error_bound_and_saturation():
    rng = np.random.default_rng(10)
    v = rng.standard_normal((32, 512)).astype(np.float32)
    codes, e8 = mx_quantize_rows(v)
    d = mx_dequantize_rows(codes, e8).astype(np.float64)
    X = np.repeat(np.exp2(e8.astype(np.float64) - 127.0), 32, axis=1)
    y = v / X
    err = np.abs(d - v)
    normal = (np.abs(y) >= 2.0 ** -6) & (np.abs(y) <= 448)
    assert np.all(err[normal] <= np.abs(v[normal]) * 2.0 ** -4 + 1e-30)   # half an ulp of 3 bits
    sub = np.abs(y) < 2.0 ** -6
    assert np.all(err[sub] <= X[sub] * 2.0 ** -10)                        # half of 2^-9
    sat = np.abs(y) > 448
    assert np.all(np.abs(d[sat]) == 448 * X[sat])


def test_sign_symmetry():
    rng = np.random.default_rng(11)
    v = rng.standard_normal((4, 96)).astype(np.float32)
    c1, e1 = mx_quantize_rows(v)
    c2, e2 = mx_quantize_rows(-v)
    assert np.array_equal(e1, e2)
    assert np.array_equal(TABLE[c2], -TABLE[c1])


def test_block_dot_identity():
    # a . b over MX blocks = sum over blocks of 2^(ea + eb) * (qa . qb), exactly
    rng = np.random.default_rng(12)
    a = rng.standard_normal((1, 128)).astype(np.float32)
    b = rng.standard_normal((1, 128)).astype(np.float32)
    ca, ea = mx_quantize_rows(a)
    cb, eb = mx_quantize_rows(b)
    lhs = float(np.dot(mx_dequantize_rows(ca, ea)[0].astype(np.float64),
                       mx_dequantize_rows(cb, eb)[0].astype(np.float64)))
    qa, qb = TABLE[ca[0]].reshape(4, 32), TABLE[cb[0]].reshape(4, 32)
    rhs = sum(2.0 ** (int(ea[0, j]) + int(eb[0, j]) - 254) * float(np.dot(qa[j], qb[j])) for j in range(4))
    assert lhs == rhs


def test_matches_the_independent_torch_conversion():
    # synth's static weight conversion (torch.frexp + torch's e4m3fn cast)
    w = torch.randn(64, 256, generator=torch.Generator().manual_seed(3)) * 0.02
    w[5, :32] = 0.0
    tc, te = _mx_rows(w)
    oc, oe = mx_quantize_rows(w.numpy())
    assert np.array_equal(te.numpy(), oe)
    assert np.array_equal(TABLE[tc.numpy()], TABLE[oc])
