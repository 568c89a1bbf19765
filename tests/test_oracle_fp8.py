"""Pins of the oracle's e4m3fn codec and block scaling (CPU only)."""
import numpy as np
import pytest
import torch

from oracle.fp8_e4m3 import (e4m3_decode, e4m3_encode, e4m3_table, quantize_groups_128,
                             dequantize_groups_128, dequantize_blocks_128x128)


def test_decode_all_codes_match_library_cast():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], lib[~nan])
    # -0 keeps its sign
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_decode_closed_form_landmarks():
    # Landmarks fixed by the E4M3 definition (bias 7, 3 mantissa bits).
    t = e4m3_table()
    assert t[0x7E] == 448.0                      # largest finite: 2^8 * 1.75
    assert t[0x01] == 2.0 ** -9                  # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9              # largest subnormal
    assert t[0x08] == 2.0 ** -6                  # smallest normal
    assert t[0x38] == 1.0 and t[0xB8] == -1.0
    assert t[0x39] == 1.125                      # 1 ulp above 1
    finite = t[np.isfinite(t)]
    assert finite.max() == 448.0 and finite.min() == -448.0


def _nearest_even_bruteforce(v):
    """Brute force: the finite code whose value is nearest; ties to the even code."""
    t = e4m3_table().astype(np.float64)
    pos = [c for c in range(0x7F) if np.isfinite(t[c])]   # non-negative codes 0x00..0x7E
    out = []
    for x in np.asarray(v, dtype=np.float64):
        a = min(abs(x), 448.0)
        d = [abs(a - t[c]) for c in pos]
        m = min(d)
        cands = [c for c, di in zip(pos, d) if di == m]
        c = min(cands, key=lambda c: (c & 1, c))
        out.append(c | (0x80 if np.signbit(x) else 0))
    return np.array(out, dtype=np.uint8)


def test_encode_matches_bruteforce_including_midpoints():
    t = e4m3_table().astype(np.float64)
    pos = np.array([t[c] for c in range(0x7F)])
    mids = (pos[:-1] + pos[1:]) / 2
    rng = np.random.default_rng(0)
    vals = np.concatenate([pos, mids, -mids, rng.uniform(-460, 460, 2000),
                           rng.standard_normal(2000) * 0.01, [0.0, -0.0, 500.0, -1e30]]).astype(np.float32)
    assert np.array_equal(e4m3_encode(vals), _nearest_even_bruteforce(vals))


def test_encode_matches_library_cast_in_range():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.uniform(-448, 448, 200000), rng.standard_normal(200000),
                        rng.standard_normal(200000) * 2.0 ** -7]).astype(np.float32)
    lib = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(v), lib)


def test_encode_saturates():
    assert e4m3_encode(np.array([448.0, 449.0, 464.0, 1e6], np.float32)).tolist() == [0x7E] * 4
    assert e4m3_encode(np.array([-1e6], np.float32)).tolist() == [0xFE]


def test_quantize_groups_scale_and_error():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((5, 384)).astype(np.float32)
    v[3, 128:256] = 0.0
    codes, scales = quantize_groups_128(v)
    assert codes.shape == (5, 384) and scales.shape == (5, 3) and scales.dtype == np.float32
    g = v.reshape(5, 3, 128)
    amax = np.abs(g).max(-1)
    exp = np.where(amax == 0, 1.0, amax / np.float32(448.0)).astype(np.float32)
    assert np.array_equal(scales, exp)
    assert scales[3, 1] == 1.0 and np.all(codes[3, 128:256] == 0)
    # the group maximum maps to +-448
    arg = np.abs(g).argmax(-1)
    for r in range(5):
        for b in range(3):
            if amax[r, b] > 0:
                assert codes[r, b * 128 + arg[r, b]] & 0x7F == 0x7E
    back = dequantize_groups_128(codes, scales)
    # relative error of e4m3 RNE for normal values is <= 2^-4; subnormal abs error <= 2^-10*scale
    err = np.abs(back - v)
    bound = np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** -10 * np.repeat(scales, 128, axis=1)) * 1.0001
    assert np.all(err <= bound)


def test_block_scaled_dot_identity():
    """sum over 128-K blocks of sa*sb*(qa . qb) equals the dot of the dequantised operands."""
    rng = np.random.default_rng(3)
    N, K = 256, 384
    wq = rng.integers(0, 256, (N, K), dtype=np.uint8)
    wq[(wq & 0x7F) == 0x7F] = 0x00           # no NaN codes
    ws = rng.uniform(1e-4, 1e-2, (N // 128, K // 128)).astype(np.float32)
    aq = rng.integers(0, 256, (K,), dtype=np.uint8)
    aq[(aq & 0x7F) == 0x7F] = 0x01
    as_ = rng.uniform(1e-3, 1.0, (K // 128,)).astype(np.float32)
    W = dequantize_blocks_128x128(wq, ws).astype(np.float64)
    a = (e4m3_decode(aq).astype(np.float64) * np.repeat(as_, 128))
    ref = W @ a
    tq = e4m3_decode(wq).astype(np.float64)
    ta = e4m3_decode(aq).astype(np.float64)
    blk = np.zeros(N)
    for n in range(N):
        for kb in range(K // 128):
            s = slice(kb * 128, kb * 128 + 128)
            blk[n] += float(ws[n // 128, kb]) * float(as_[kb]) * float(tq[n, s] @ ta[s])
    # dequantised fp32 weights carry one fp32 rounding each: bound by sum |terms| * 2^-23
    mag = np.abs(tq * np.repeat(np.repeat(ws, 128, 0), 128, 1)) @ np.abs(a)
    assert np.all(np.abs(ref - blk) <= mag * 2.0 ** -23)
