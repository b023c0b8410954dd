"""Pins of the oracle's mixed-precision entry store (the decode cache layout:
the 64 RoPE dims kept in BF16, the other 64 dims in FP8 e4m3 with one fp32
scale per row), "DeepSeek-V4: Towards Highly Efficient Million-Token Context
Intelligence" wiki summary, Training infrastructure item 5.

The store under test is ``oracle.store_entries_fp8(rows, rope_dims=64)`` and
its inverse ``oracle.load_entries_fp8``.  Every expected value here comes
from an independent route:
  * the e4m3 value table is built in this file from the OCP bit layout
    (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, 0x7f/0xff NaN);
  * each code is checked as a nearest grid value by brute force over all
    finite codes (ties to the even mantissa, saturating at 448, results of
    zero stored as +0);
  * the scale is amax(dims 0..63) / 448 in numpy fp32 (IEEE division);
  * dims 64..127 are torch's bf16 cast (round to nearest even).
A mistake such as an amax over all 128 dims, the FP8 and BF16 halves
swapped, or the scale applied the wrong way round fails one of them.
"""
import numpy as np
import pytest
import torch

import oracle


def _e4m3_table():
    """Value of every positive finite e4m3fn code 0x00 .. 0x7e."""
    vals = np.empty(127, np.float64)
    for c in range(127):
        e, m = (c >> 3) & 15, c & 7
        vals[c] = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return vals


E4M3 = _e4m3_table()


def _nearest_code(v):
    """Brute force: the code of the finite e4m3 value nearest to fp32 v,
    ties to the even code; values that round to 0 give +0."""
    a = abs(float(v))
    d = np.abs(E4M3 - a)
    best = np.flatnonzero(d == d.min())
    c = int(best[0]) if best.size == 1 else int(best[best % 2 == 0][0])
    if c == 0:
        return 0
    return c | (0x80 if v < 0 else 0)


def _bf16_bits_torch(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def _rows(seed, n=40):
    rng = np.random.default_rng(seed)
    r = rng.standard_normal((n, 128)).astype(np.float32)
    # the RoPE half much larger than the FP8 half on some rows, smaller on
    # others: an amax over all 128 dims would give another scale
    r[::3, 64:] *= 50.0
    r[1::3, :64] *= 7.0
    r[2::3, :64] *= 1e-3
    return r


def test_table_is_the_ocp_grid():
    assert E4M3[0x7e] == 448.0 and E4M3[0x08] == 2.0 ** -6 and E4M3[0x01] == 2.0 ** -9
    assert np.all(np.diff(E4M3) > 0)
    # the oracle's decoder agrees with the table on every finite code and sign
    codes = np.array([c for c in range(256) if (c & 0x7f) != 0x7f], np.uint8)
    dec = oracle.e4m3_to_f32(codes).astype(np.float64)
    want = np.where(codes & 0x80, -1.0, 1.0) * E4M3[codes & 0x7f]
    assert np.array_equal(dec, want)


def test_scale_is_amax_of_the_fp8_dims_only():
    rows = _rows(1)
    _, _, scale = oracle.store_entries_fp8(rows, rope_dims=64)
    want = (np.abs(rows[:, :64]).max(axis=1).astype(np.float32) / np.float32(448.0)).astype(np.float32)
    assert scale.dtype == np.float32
    assert np.array_equal(scale, want)
    wrong = np.abs(rows).max(axis=1).astype(np.float32) / np.float32(448.0)
    assert np.any(wrong != want)  # the fixture tells the two readings apart


def test_rope_dims_are_exact_bf16():
    rows = _rows(2)
    _, rope, _ = oracle.store_entries_fp8(rows, rope_dims=64)
    assert rope.shape == (rows.shape[0], 64)
    assert np.array_equal(rope, _bf16_bits_torch(rows[:, 64:]))


def test_codes_are_nearest_e4m3_of_x_over_scale():
    rows = _rows(3, n=24)
    codes, _, scale = oracle.store_entries_fp8(rows, rope_dims=64)
    assert codes.shape == (rows.shape[0], 64)
    for i in range(rows.shape[0]):
        v = (rows[i, :64] / scale[i]).astype(np.float32)  # fp32 IEEE division
        want = np.array([_nearest_code(x) for x in v], np.uint8)
        assert np.array_equal(codes[i], want), i
        # the largest element codes to +-448 exactly
        j = int(np.argmax(np.abs(rows[i, :64])))
        assert codes[i, j] & 0x7f == 0x7e


def test_round_trip_within_half_a_step():
    rows = _rows(4)
    codes, rope, scale = oracle.store_entries_fp8(rows, rope_dims=64)
    back = oracle.load_entries_fp8(codes, rope, scale)
    assert back.shape == rows.shape
    x = rows[:, :64].astype(np.float64)
    a = np.abs(x) / scale[:, None]
    # e4m3 spacing at |x|/scale: 2^(floor(log2 a) - 3), 2^-9 below 2^-6
    k = np.floor(np.log2(np.maximum(a, 2.0 ** -30)))
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (k - 3))
    err = np.abs(back[:, :64] - x)
    assert np.all(err <= step / 2 * scale[:, None] * (1 + 1e-6) + 1e-30)
    # the RoPE half comes back as the bf16 values
    assert np.array_equal(back[:, 64:], oracle.bf16_to_f64(_bf16_bits_torch(rows[:, 64:])))


def test_hand_worked_row():
    """amax = 448 gives scale 1, so the codes are the e4m3 codes of the
    values themselves:
      448      -> 0x7e (the largest finite value)
      1.0625   -> a tie between 1 and 1.125: the even mantissa, 1.0 = 0x38
      -3.1     -> nearest 3.0 = (1 + 4/8) 2^1: 0x80 | (8 << 3) | 4 = 0xc4
      2^-10    -> a tie between 0 and 2^-9: the even code, +0
      -2^-11   -> rounds to zero: +0, not -0
      0.3      -> binade [0.25, 0.5), step 2^-5: 0.3125 = (1 + 2/8) 2^-2 = 0x2a
    dims 64..127 hold 1000.5, which bf16 rounds to 1000 (8 bits of
    mantissa: spacing 4 in [512, 1024); 1000.5 is nearer to 1000)."""
    row = np.zeros((1, 128), np.float32)
    row[0, :6] = [448.0, 1.0625, -3.1, 2.0 ** -10, -(2.0 ** -11), 0.3]
    row[0, 64:] = 1000.5
    codes, rope, scale = oracle.store_entries_fp8(row, rope_dims=64)
    assert scale[0] == np.float32(1.0)
    assert list(codes[0, :6]) == [0x7e, 0x38, 0xc4, 0x00, 0x00, 0x2a]
    assert np.all(codes[0, 6:] == 0)
    assert np.all(oracle.bf16_to_f64(rope[0]) == 1000.0)


def test_zero_fp8_half_keeps_the_rope_half():
    row = np.zeros((2, 128), np.float32)
    row[:, 64:] = np.linspace(-3, 3, 64, dtype=np.float32)
    codes, rope, scale = oracle.store_entries_fp8(row, rope_dims=64)
    assert np.all(scale == 0) and np.all(codes == 0)
    assert np.array_equal(rope, _bf16_bits_torch(row[:, 64:]))
    back = oracle.load_entries_fp8(codes, rope, scale)
    assert np.all(back[:, :64] == 0)


@pytest.mark.parametrize("p", [-8, 0, 9])
def test_power_of_two_scaling_scales_only_the_scale(p):
    """Multiplying a row by 2^p multiplies the scale by 2^p exactly and
    leaves every FP8 code unchanged (the division x / scale is exact in
    the same ratio); the bf16 half scales exactly too."""
    rows = _rows(5, n=12)
    c0, r0, s0 = oracle.store_entries_fp8(rows, rope_dims=64)
    c1, r1, s1 = oracle.store_entries_fp8((rows * np.float32(2.0 ** p)).astype(np.float32), rope_dims=64)
    assert np.array_equal(c0, c1)
    assert np.array_equal(s1, (s0 * np.float32(2.0 ** p)).astype(np.float32))
    assert np.array_equal(oracle.bf16_to_f64(r1), oracle.bf16_to_f64(r0) * 2.0 ** p)


def test_sign_symmetry():
    rows = _rows(6, n=12)
    c0, r0, s0 = oracle.store_entries_fp8(rows, rope_dims=64)
    c1, r1, s1 = oracle.store_entries_fp8(-rows, rope_dims=64)
    assert np.array_equal(s0, s1)
    nz = (c0 & 0x7f) != 0
    assert np.array_equal(c1[nz], c0[nz] ^ 0x80) and np.all(c1[~nz] == 0)
    assert np.array_equal(oracle.bf16_to_f64(r1), -oracle.bf16_to_f64(r0))
