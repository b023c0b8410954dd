"""Pins of the oracle's NVFP4 entry storage (the V4.1 cache variant: the
Russian summary of DeepSeek-V4.1-Flash stores the compressed KV cache in
NVFP4, quantised after RoPE).  NVFP4 is e2m1 elements in blocks of 16 with
an e4m3 block scale and an fp32 second-level scale (here per entry,
amax / (6 * 448)).  Pinned against values built exactly on the grids, the
rounding rule checked by brute force over the 8 e2m1 magnitudes, hand
worked ties and saturation, power-of-two scaling and sign symmetry.  Also
the FP8 sliding-window cache of the same variant (rows rotated at their
position, then e4m3 over all 128 dims with scale amax / 448)."""
import numpy as np
import pytest

import oracle

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _codes(rec):
    """[.., 72] records -> [.., 128] e2m1 codes (dim 2i low nibble)."""
    lo, hi = rec[..., :64] & 15, rec[..., :64] >> 4
    return np.stack([lo, hi], axis=-1).reshape(rec.shape[:-1] + (128,))


def _e4m3(code):
    return np.array([oracle.e4m3_to_f32(np.array([c], np.uint8))[0] for c in np.ravel(code)]).reshape(np.shape(code))


def test_grid_values_round_trip_exactly():
    """An entry whose block maxima are 6 x (an e4m3 value) x s and whose
    elements lie on e2m1 x (that e4m3 value) x s is stored exactly."""
    rng = np.random.default_rng(1)
    s = 2.0 ** -10                      # amax = 6 * 448 * s = 2.625
    bvals = [448.0, 1.0, 0.5, 96.0, 3.25, 0.015625, 12.0, 240.0]
    x = np.zeros(128)
    for j, bv in enumerate(bvals):
        mags = E2M1[rng.integers(0, 8, 16)]
        mags[rng.integers(0, 16)] = 6.0  # the block maximum
        signs = np.where(rng.random(16) < 0.5, -1.0, 1.0)
        x[16 * j:16 * j + 16] = signs * mags * bv * s
    rec, sc = oracle.store_entries_nvfp4(x.astype(np.float32)[None])
    assert sc[0] == np.float32(s)
    assert np.array_equal(_e4m3(rec[0, 64:]), np.array(bvals))
    assert np.array_equal(oracle.load_entries_nvfp4(rec, sc)[0], x)


def test_rounding_is_nearest_on_the_grid_brute_force():
    """Every element's code is a nearest e2m1 magnitude of x / (b s) (the
    block scale and s as stored), ties to the even code, saturating at 6."""
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((64, 128)) * np.exp(rng.uniform(-4, 4, (64, 1)))).astype(np.float32)
    rec, sc = oracle.store_entries_nvfp4(x)
    codes = _codes(rec)
    for r in range(x.shape[0]):
        b = _e4m3(rec[r, 64:])
        for d in range(128):
            sb = np.float32(np.float32(b[d // 16]) * sc[r])
            q = abs(float(np.float32(x[r, d] / sb)))
            dist = np.abs(E2M1 - min(q, 6.0))
            best = np.flatnonzero(dist == dist.min())
            c = int(codes[r, d]) & 7
            assert c in best and (len(best) == 1 or c % 2 == 0), (r, d, q, c)
            assert (int(codes[r, d]) >> 3) == (1 if (x[r, d] < 0 and c != 0) else 0)


def test_block_scale_rule():
    """b_j = e4m3(amax_j / (6 s)) with s = amax / 2688, every step in fp32."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((32, 128)) * rng.uniform(0.01, 50, (32, 1))).astype(np.float32)
    rec, sc = oracle.store_entries_nvfp4(x)
    amax = np.abs(x).max(axis=1)
    assert np.array_equal(sc, (amax / np.float32(2688.0)).astype(np.float32))
    for r in range(32):
        d6 = np.float32(np.float32(6.0) * sc[r])
        t = (np.abs(x[r]).reshape(8, 16).max(axis=1) / d6).astype(np.float32)
        assert np.array_equal(rec[r, 64:], oracle.e4m3_from_f32(t))
    # the block holding the entry's maximum gets 448
    j = np.abs(x).argmax(axis=1) // 16
    assert np.all(_e4m3(rec[np.arange(32), 64 + j]) == 448.0)


def test_hand_worked_ties_and_saturation():
    """s = 2^-10 (amax 2.625 in block 0).  Block 1: amax 1.0625 x 6 s gives
    t = 1.0625, a tie between the e4m3 values 1 and 1.125 -> 1 (even
    mantissa); its maximum then divides to 6.375 and saturates to 6.  Block 2
    (b = 448): x / (448 s) = 2.5 ties between 2 and 3 -> 2; 0.25 ties between
    0 and 0.5 -> 0; 5 ties between 4 and 6 -> 4; 1.25 ties between 1 and 1.5
    -> 1; -0.75 ties between -0.5 and -1 -> -1 (index 2 is even)."""
    s = 2.0 ** -10
    x = np.zeros(128)
    x[0] = 6 * 448 * s
    x[16] = 1.0625 * 6 * s
    x[17] = -0.5 * s                       # / (1 * s) = -0.5 exactly
    x[32:38] = np.array([6.0, 2.5, 0.25, 5.0, 1.25, -0.75]) * 448 * s
    rec, sc = oracle.store_entries_nvfp4(x.astype(np.float32)[None])
    c = _codes(rec)[0]
    assert sc[0] == np.float32(s)
    assert _e4m3(rec[0, 65]) == 1.0 and _e4m3(rec[0, 66]) == 448.0
    assert c[16] == 7 and c[17] == 8 | 1
    assert list(c[32:38]) == [7, 4, 0, 6, 2, 8 | 2]
    assert not c[38:48].any() and not c[48:].any() and not rec[0, 67:].any()


def test_zero_and_flushed_blocks():
    x = np.zeros((2, 128), np.float32)
    x[1, 0] = 1000.0
    x[1, 16:32] = 1e-6                     # amax_j / (6 s) below the e4m3 subnormal half-step
    rec, sc = oracle.store_entries_nvfp4(x)
    assert sc[0] == 0 and not rec[0].any()
    assert rec[1, 65] == 0 and not _codes(rec)[1, 16:32].any()
    assert not oracle.load_entries_nvfp4(rec, sc)[0].any()


def test_power_of_two_scaling_and_sign_symmetry():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((16, 128)).astype(np.float32)
    rec, sc = oracle.store_entries_nvfp4(x)
    for k in (-7, 3, 11):
        r2, s2 = oracle.store_entries_nvfp4(np.ldexp(x, k))
        assert np.array_equal(r2, rec) and np.array_equal(s2, np.ldexp(sc, k))
    rn, sn = oracle.store_entries_nvfp4(-x)
    c, cn = _codes(rec), _codes(rn)
    assert np.array_equal(sn, sc) and np.array_equal(rn[:, 64:], rec[:, 64:])
    nz = (c & 7) != 0
    assert np.array_equal(cn[nz], c[nz] ^ 8) and np.array_equal(cn[~nz], c[~nz])


@pytest.mark.parametrize("seed", [5, 6])
def test_error_bound(seed):
    """|x - x_hat| <= half the e2m1 spacing at |x| / (b s), times b s, for
    unsaturated elements (spacing 0.5 below 2, 1 below 4, 2 above)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((128, 128)).astype(np.float32)
    rec, sc = oracle.store_entries_nvfp4(x)
    xh = oracle.load_entries_nvfp4(rec, sc)
    b = _e4m3(rec[:, 64:]).repeat(16, axis=1)
    sb = b * sc[:, None].astype(np.float64)
    q = np.abs(x) / np.where(sb > 0, sb, 1)
    spacing = np.where(q < 2, 0.5, np.where(q < 4, 1.0, 2.0))
    ok = (q <= 6) & (sb > 0)
    err = np.abs(x - xh)
    assert np.all(err[ok] <= spacing[ok] / 2 * sb[ok] * (1 + 1e-6))


# ---- the FP8 sliding-window cache of the V4.1 variant ----------------------

def _raw_rows(rng, n, scale=0.5):
    return oracle.bf16_from_f32((rng.standard_normal((n, 128)) * scale).astype(np.float32))


def test_window_fp8_at_position_zero_is_plain_fp8():
    """RoPE at position 0 is the identity, so row 0 is the FP8 entry rule
    over all 128 dims (scale amax / 448)."""
    rng = np.random.default_rng(10)
    w = _raw_rows(rng, 3)
    codes, sc = oracle.store_window_fp8(w, 0)
    c0, _, s0 = oracle.store_entries_fp8(oracle.bf16_to_f64(w[:1]).astype(np.float32), rope_dims=0)
    assert np.array_equal(codes[0], c0[0]) and sc[0] == s0[0]
    assert sc[0] == np.float32(np.abs(oracle.bf16_to_f64(w[0])).max()) / np.float32(448.0)


def test_window_fp8_is_the_rotated_row_within_fp8_error():
    rng = np.random.default_rng(11)
    pos0 = 1_000_000
    w = _raw_rows(rng, 64)
    codes, sc = oracle.store_window_fp8(w, pos0)
    dec = oracle.load_window_fp8(codes, sc)
    for i in range(64):
        rot = oracle.bf16_to_f64(w[i]).copy()
        rot = oracle.rope(rot, pos0 + i)
        assert np.all(np.abs(dec[i] - rot) <= 2.0 ** -4 * np.abs(rot) + float(sc[i]) * 2.0 ** -9)
        # the rotation keeps each (2f, 2f+1) pair's length: dims 0..63 are not rotated
        assert np.allclose(np.hypot(rot[64::2], rot[65::2]),
                           np.hypot(*oracle.bf16_to_f64(w[i])[64:].reshape(32, 2).T), rtol=1e-12)


def test_attention_over_a_rotated_window_equals_the_raw_window():
    """The post-RoPE window input (used for the FP8 cache) and the raw one
    give the same attention when the post-RoPE rows are the exact rotations."""
    rng = np.random.default_rng(12)
    H, n, pos0 = 8, 6, 300
    q = oracle.bf16_from_f32((rng.standard_normal((n, H, 128)) * 0.3).astype(np.float32))
    win = _raw_rows(rng, pos0 + n, 0.3)
    post = np.stack([oracle.rope(oracle.bf16_to_f64(win[j]).copy(), j) for j in range(pos0 + n)])
    ent = rng.standard_normal((75, 128))
    rows = np.arange(n, dtype=np.int32)
    idx = np.sort(rng.choice(75, size=(n, 20)), axis=1).astype(np.int32)
    sink = rng.standard_normal(H).astype(np.float32)
    a = oracle.attend_rows(q, pos0, ent, 4, rows, "csa", idx=idx, win=win, sink=sink)
    b = oracle.attend_rows(q, pos0, ent, 4, rows, "csa", idx=idx, win_post=post, sink=sink)
    assert np.array_equal(a, b)
