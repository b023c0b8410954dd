"""Pins for the CPU oracle: each test checks it against something other than
itself -- a library routine (torch casts, torch SDPA, complex
multiplication), a closed form, an invariant, or the independent fp64
brute-force construction in oracle/bruteforce.py.  The pages print no worked
numeric example, so no golden values from them exist; tests/golden holds
the tables of the OCP formats used here (see tests/golden/README.md).

CPU only.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bruteforce as bf


def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


# ---------------------------------------------------------------- formats --

def test_bf16_rne_matches_torch(orc):
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(10.0) ** rng.integers(-20, 20, 200000).astype(np.float32)
    # exact halfway cases: low 16 bits = 0x8000, both parities of bit 16
    hw = (rng.integers(0, 2**31, 5000, dtype=np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = np.concatenate([x, hw.view(np.float32), np.array([0.0, -0.0, 65504.0, 3.4e38, -3.4e38], np.float32)])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.bf16_from_f32(x), ref)


def test_e4m3_decode_exhaustive_vs_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = orc.e4m3_to_f32(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.nanmax(got) == 448.0


def test_e4m3_encode_vs_torch_in_range(orc):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100000) * 2.0 ** rng.integers(-12, 9, 100000)).astype(np.float32)
    x = np.clip(x, -448, 448)
    # every midpoint between adjacent finite codes (ties-to-even cases)
    vals = np.unique(np.abs(orc.e4m3_to_f32(np.arange(0, 0x7F, dtype=np.uint8))))
    mids = ((vals[1:].astype(np.float64) + vals[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, vals, -vals])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.e4m3_from_f32(x)
    # torch keeps the sign of zero; the oracle canonicalises zero to +0
    ref = np.where((ref & 0x7F) == 0, 0, ref).astype(np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_saturates(orc):
    x = np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e9, -1e9], np.float32)
    got = orc.e4m3_to_f32(orc.e4m3_from_f32(x))
    assert np.array_equal(np.abs(got), np.full(7, 448.0, np.float32))


def test_e2m1_table_matches_ocp_fields(orc):
    # OCP MX v1.0: e2m1 = sign | 2-bit exponent (bias 1) | 1-bit mantissa.
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        v = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        if s:
            v = -v
        codes = np.array([code | (code << 4)] * 16, np.uint8)
        got = orc.mxfp4_decode(codes, np.array([127], np.uint8))
        assert got[0] == v and got[1] == v


def test_e2m1_table_golden(orc):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "e2m1_values.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    for code_s, val_s in rows:
        code = int(code_s, 16)
        codes = np.array([code] * 16, np.uint8)
        got = orc.mxfp4_decode(codes, np.array([127], np.uint8))[0]
        assert got == float(val_s)


def test_mxfp4_encode_rules(orc):
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((4000, 32)) * 2.0 ** rng.integers(-20, 20, (4000, 1))).astype(np.float32)
    codes, scales = orc.mxfp4_encode(x)
    dec = orc.mxfp4_decode(codes, scales)
    E = scales.astype(np.int64)[:, 0] - 127
    amax = np.abs(x).max(axis=1).astype(np.float64)
    # shared scale: amax in [4 * 2^E, 8 * 2^E)  (E = floor(log2 amax) - 2)
    assert np.all(amax >= 4 * 2.0 ** E) and np.all(amax < 8 * 2.0 ** E)
    # error: within half a grid step of the nearest grid value, except clipping above 6*2^E
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    for r in range(200):
        sc = 2.0 ** E[r]
        for i in range(32):
            a = abs(float(x[r, i])) / sc
            g = grid[np.argmin(np.abs(grid - min(a, 6.0)))]
            assert abs(abs(float(dec[r, i])) / sc - g) <= 1e-12 or abs(abs(a - g) - abs(a - abs(float(dec[r, i])) / sc)) <= 1e-12


def test_mxfp4_roundtrip_and_ties(orc):
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    # on-grid values round-trip exactly (block amax 6 -> E = 0)
    x = np.concatenate([grid, -grid[1:], grid[:8], grid[:1], [6.0] * 8]).astype(np.float32)[:32]
    c, s = orc.mxfp4_encode(x[None])
    assert s[0, 0] == 127
    assert np.array_equal(orc.mxfp4_decode(c, s)[0], x)
    # midpoints go to the even code: 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    want = np.array([0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0], np.float32)
    blk = np.zeros(32, np.float32)
    blk[:7] = mids
    blk[31] = 6.0
    c, s = orc.mxfp4_encode(blk[None])
    assert np.array_equal(orc.mxfp4_decode(c, s)[0, :7], want)
    # all-zero block
    c, s = orc.mxfp4_encode(np.zeros((1, 32), np.float32))
    assert s[0, 0] == 0 and not c.any()


def test_fp4_to_fp8_lossless(orc):
    """FP4 -> FP8 dequantisation is lossless [V4-wiki, Post-training item 3]:
    every e2m1 value times 2^E (E in the range e4m3 covers) is an e4m3 value."""
    vals = np.array([0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    for E in range(-8, 7):
        x = (vals * 2.0 ** E).astype(np.float32)
        back = orc.e4m3_to_f32(orc.e4m3_from_f32(x))
        assert np.array_equal(back, x), E


# ------------------------------------------------------------------- RoPE --

def test_rope_is_complex_multiplication(orc):
    rng = np.random.default_rng(3)
    for pos in [0, 1, 7, 1000, 1048575, 1056767]:
        v = rng.standard_normal(128)
        got = orc.rope(v, pos)
        z = v[64::2] + 1j * v[65::2]
        f = np.arange(32)
        z = z * np.exp(1j * (pos * 10000.0 ** (-f / 32.0)))
        ref = v.copy()
        ref[64::2], ref[65::2] = z.real, z.imag
        # the angle is pos * theta in fp64: an ulp of theta moves it by ~pos * 1e-16
        assert np.allclose(got, ref, rtol=0, atol=1e-12 + pos * 1e-15)
        assert np.array_equal(got[:64], v[:64])
        assert math.isclose(np.linalg.norm(got), np.linalg.norm(v), rel_tol=1e-13)
        back = orc.rope(got, -pos)
        assert np.allclose(back, v, atol=1e-12)


# ------------------------------------------------------------ compression --

def _rand_bf16(rng, shape, scale=1.0):
    return torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("m,overlap,with_z", [(4, 1, False), (4, 1, True), (8, 0, True), (4, 0, False)])
def test_compress_vs_bruteforce(orc, m, overlap, with_z):
    rng = np.random.default_rng(4)
    T = 13 * m + 3
    kv = _rand_bf16(rng, (T, 128), 0.1)
    ik = _rand_bf16(rng, (T, 64), 0.1)
    beta = rng.standard_normal(2 * m if overlap else m).astype(np.float32)
    z = rng.standard_normal((T, 2)).astype(np.float32) if with_z else None
    ent, kid = orc.compress(kv, beta, m, overlap, ik=ik, z=z)
    C, E = bf.compress(kv, beta, m, overlap, ik_bits=ik, z=z)
    assert ent.shape == (T // m, 128)
    assert np.allclose(ent, C, rtol=0, atol=1e-6)
    assert np.allclose(kid, E, rtol=0, atol=1e-6)


def test_compress_equal_logits_is_mean(orc):
    rng = np.random.default_rng(5)
    T, m = 40, 4
    kv = _rand_bf16(rng, (T, 128))
    X = bf.bf16_bits_to_f64(kv)
    ent, _ = orc.compress(kv, np.zeros(8, np.float32), m, 1, rope_dims=0)
    for i in range(T // m):
        lo = max(0, (i - 1) * m)
        assert np.allclose(ent[i], X[lo:(i + 1) * m].mean(axis=0), atol=1e-6)


@pytest.mark.parametrize("slot", range(8))
def test_compress_dominant_slot_copies_its_token(orc, slot):
    """Overlap geometry: slot r < m is token (i-1)m + r (previous block),
    slot r >= m is token im + r - m (current block)."""
    rng = np.random.default_rng(6)
    T, m = 32, 4
    kv = _rand_bf16(rng, (T, 128))
    X = bf.bf16_bits_to_f64(kv)
    beta = np.zeros(8, np.float32)
    beta[slot] = 200.0
    ent, _ = orc.compress(kv, beta, m, 1, rope_dims=0)
    for i in range(1, T // m):
        j = (i - 1) * m + slot if slot < m else i * m + slot - m
        assert np.array_equal(ent[i], X[j].astype(np.float32))


def test_compress_identity_and_constants(orc):
    rng = np.random.default_rng(7)
    kv = _rand_bf16(rng, (50, 128))
    ent, _ = orc.compress(kv, np.zeros(1, np.float32), 1, 0, rope_dims=0)
    assert np.array_equal(ent, bf.bf16_bits_to_f64(kv).astype(np.float32))
    const = np.full((64, 128), 0x3FC0, np.uint16)  # 1.5
    ent, _ = orc.compress(const, rng.standard_normal(8).astype(np.float32), 4, 1, rope_dims=0)
    assert np.allclose(ent, 1.5, atol=1e-6)


def test_compress_chunked_matches_whole(orc):
    """Compressing a chunk with the previous block passed as prev_* gives the
    same entries as one pass over the whole sequence."""
    rng = np.random.default_rng(8)
    T, m = 96, 4
    kv = _rand_bf16(rng, (T, 128))
    ik = _rand_bf16(rng, (T, 64))
    z = rng.standard_normal((T, 2)).astype(np.float32)
    beta = rng.standard_normal(8).astype(np.float32)
    whole, wk = orc.compress(kv, beta, m, 1, ik=ik, z=z)
    p0 = 40
    part, pk = orc.compress(kv[p0:], beta, m, 1, pos0=p0, ik=ik[p0:], z=z[p0:],
                            prev_kv=kv[p0 - m:p0], prev_ik=ik[p0 - m:p0], prev_z=z[p0 - m:p0])
    assert np.array_equal(part, whole[p0 // m:])
    assert np.array_equal(pk, wk[p0 // m:])


# ---------------------------------------------------------- indexer / top-k --

def test_index_scores_fp4_dot_exact(orc):
    """With MXFP4 operands every dot product is exact in fp32; check it
    against exact rational arithmetic (single head, w = 1)."""
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 64)).astype(np.float32)
    keys = (rng.standard_normal((300, 64)) * 2.0 ** rng.integers(-3, 3, (300, 1))).astype(np.float32)
    qc, qs = orc.mxfp4_encode(q)
    kc, ks = orc.mxfp4_encode(keys)
    qd = orc.mxfp4_decode(qc, qs)
    kd = orc.mxfp4_decode(kc, ks)
    got = orc.index_scores(qd, np.ones(1, np.float32), kd, relu=False)
    for s in range(300):
        exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qd[0], kd[s]))
        assert Fraction(float(got[s])) == exact


def test_index_scores_vs_bruteforce(orc):
    rng = np.random.default_rng(10)
    q = rng.standard_normal((8, 64)).astype(np.float32) / 8
    w = rng.standard_normal(8).astype(np.float32)
    keys = rng.standard_normal((500, 64)).astype(np.float32) / 8
    got = orc.index_scores(q, w, keys)
    ref = bf.index_scores(q[None].astype(np.float64), w[None].astype(np.float64), keys.astype(np.float64))[0]
    assert np.allclose(got, ref, rtol=1e-5, atol=1e-6)
    # relu matters: without it the scores differ
    assert not np.allclose(orc.index_scores(q, w, keys, relu=False), got)


@pytest.mark.parametrize("k", [1, 3, 50, 200, 205])
def test_topk_vs_full_sort(orc, k):
    rng = np.random.default_rng(11)
    for trial in range(20):
        n = int(rng.integers(1, 201))
        s = np.round(rng.standard_normal(n) * 4).astype(np.float32)  # many ties
        got = orc.topk(s, k)
        ref = bf.topk_rows(s[None].astype(np.float64), [n], k)[0]
        assert np.array_equal(got, ref)


# --------------------------------------------------------------- attention --

def _sdpa_causal(qf, kf, t0=0):
    """Causal softmax attention with one shared K=V head, via torch SDPA (fp64)."""
    n, H, D = qf.shape
    q = torch.from_numpy(qf).permute(1, 0, 2)[None]
    k = torch.from_numpy(kf)[None, None].expand(1, H, -1, D)
    return torch.nn.functional.scaled_dot_product_attention(q, k, k, is_causal=True)[0].permute(1, 0, 2).numpy()


def test_attention_reduces_to_causal_sdpa(orc):
    """m = 1, no overlap, top-k = all, no window, no sink, no RoPE: exactly
    causal softmax attention with K = V = the token rows."""
    rng = np.random.default_rng(12)
    n, H = 40, 4
    q = _rand_bf16(rng, (n, H, 128), 0.5)
    kv = _rand_bf16(rng, (n, 128), 0.5)
    ent, _ = orc.compress(kv, np.zeros(1, np.float32), 1, 0, rope_dims=0)
    rows = np.arange(n, dtype=np.int32)
    idx = np.full((n, n), -1, np.int32)
    for t in range(n):
        idx[t, :t + 1] = np.arange(t + 1)
    got = orc.attend_rows(q, 0, ent.astype(np.float64), 1, rows, "csa", idx=idx, rope_dims=0)
    ref = _sdpa_causal(bf.bf16_bits_to_f64(q), bf.bf16_bits_to_f64(kv))
    assert np.allclose(got, ref, atol=1e-12)
    # window over the whole sequence duplicates every key: unchanged result
    got2 = orc.attend_rows(q, 0, ent.astype(np.float64), 1, rows, "csa", idx=idx, win=kv,
                           n_win=n, rope_dims=0)
    assert np.allclose(got2, ref, atol=1e-12)
    # HCA mode (all visible entries) is the same thing
    got3 = orc.attend_rows(q, 0, ent.astype(np.float64), 1, rows, "hca", rope_dims=0)
    assert np.allclose(got3, ref, atol=1e-12)


def test_attention_with_rope_matches_sdpa_on_rotated_inputs(orc):
    rng = np.random.default_rng(13)
    n, H = 33, 3
    q = _rand_bf16(rng, (n, H, 128), 0.5)
    kv = _rand_bf16(rng, (n, 128), 0.5)
    ent, _ = orc.compress(kv, np.zeros(1, np.float32), 1, 0)  # rotates entry i at p = i
    rows = np.arange(n, dtype=np.int32)
    got = orc.attend_rows(q, 0, ent.astype(np.float64), 1, rows, "hca")
    qr = bf.rope_complex(bf.bf16_bits_to_f64(q), np.arange(n)[:, None])
    kr = bf.rope_complex(bf.bf16_bits_to_f64(kv), np.arange(n))
    ref = bf.rope_complex(_sdpa_causal(qr, kr), np.arange(n)[:, None], sign=-1.0)
    assert np.allclose(got, ref, atol=2e-7)  # entries pass through fp32


def test_sink_closed_form(orc):
    """With a sink logit s0: out = (1 - p_sink) * out_without_sink, where
    p_sink = sigmoid(s0 - logsumexp(logits)); weights + sink weight = 1."""
    rng = np.random.default_rng(14)
    n, H = 20, 4
    q = _rand_bf16(rng, (n, H, 128), 2.0)
    kv = _rand_bf16(rng, (n, 128), 1.0)
    ent, _ = orc.compress(kv, np.zeros(1, np.float32), 1, 0, rope_dims=0)
    sink = rng.standard_normal(H).astype(np.float32) * 2
    rows = np.arange(n, dtype=np.int32)
    a = orc.attend_rows(q, 0, ent.astype(np.float64), 1, rows, "hca", rope_dims=0)
    b = orc.attend_rows(q, 0, ent.astype(np.float64), 1, rows, "hca", rope_dims=0, sink=sink)
    Q = torch.from_numpy(bf.bf16_bits_to_f64(q))
    K = torch.from_numpy(bf.bf16_bits_to_f64(kv))
    for t in range(n):
        lg = (Q[t] @ K[:t + 1].T) / math.sqrt(128)
        lse = torch.logsumexp(lg, dim=1).numpy()
        p_sink = 1 / (1 + np.exp(lse - sink.astype(np.float64)))
        assert np.allclose(b[t], (1 - p_sink)[:, None] * a[t], atol=1e-13)
        assert np.all(p_sink > 0) and np.all(p_sink < 1)


def test_attention_vs_bruteforce_csa_and_hca(orc):
    rng = np.random.default_rng(15)
    n, H, m = 48, 4, 4
    q = _rand_bf16(rng, (n, H, 128), 1.0)
    kv = _rand_bf16(rng, (n, 128), 0.5)
    beta = rng.standard_normal(8).astype(np.float32)
    ent, _ = orc.compress(kv, beta, m, 1)
    E = ent.astype(np.float64)
    sink = rng.standard_normal(H).astype(np.float32)
    rows = np.arange(n, dtype=np.int32)
    idx = np.full((n, 5), -1, np.int32)
    for t in range(n):
        nv = (t + 1) // m
        if nv:
            sel = np.sort(rng.choice(nv, size=min(5, nv), replace=False))
            idx[t, :sel.size] = sel
    for mode in ["csa", "hca"]:
        for n_win in [0, 1, 7, 128]:
            got = orc.attend_rows(q, 0, E, m, rows, mode, idx=idx if mode == "csa" else None,
                                  win=kv, n_win=n_win, sink=sink)
            ref = bf.attend(q, 0, E, m, mode, idx=idx, win_bits=kv, n_win=n_win, sink=sink)
            assert np.allclose(got, ref, atol=1e-12), (mode, n_win)


def test_csa_all_visible_equals_hca(orc):
    rng = np.random.default_rng(16)
    n, H, m = 64, 2, 4
    q = _rand_bf16(rng, (n, H, 128))
    kv = _rand_bf16(rng, (n, 128))
    ent, _ = orc.compress(kv, rng.standard_normal(8).astype(np.float32), m, 1)
    E = ent.astype(np.float64)
    rows = np.arange(n, dtype=np.int32)
    idx = np.full((n, 16), -1, np.int32)
    for t in range(n):
        nv = (t + 1) // m
        idx[t, :nv] = np.arange(nv)
    sink = rng.standard_normal(H).astype(np.float32)
    a = orc.attend_rows(q, 0, E, m, rows, "csa", idx=idx, win=kv, sink=sink)
    b = orc.attend_rows(q, 0, E, m, rows, "hca", win=kv, sink=sink)
    assert np.allclose(a, b, atol=1e-14)


def test_position_shift_invariance(orc):
    """Scores depend on relative positions only: shifting every position by
    a multiple of m leaves the (inverse-rotated) output unchanged."""
    rng = np.random.default_rng(17)
    n, H, m = 300, 2, 128
    q = _rand_bf16(rng, (n, H, 128))
    kv = _rand_bf16(rng, (n, 128))
    beta = rng.standard_normal(m).astype(np.float32)
    rows = np.arange(127, n, 7, dtype=np.int32)  # full windows inside the source
    sink = rng.standard_normal(H).astype(np.float32)
    outs = []
    for shift in [0, 128 * 8191]:
        ent, _ = orc.compress(kv, beta, m, 0, pos0=shift)
        e0 = shift // m
        E = np.zeros((e0 + ent.shape[0], 128))
        E[e0:] = ent
        idx = np.full((rows.size, 4), -1, np.int32)
        for r, qrow in enumerate(rows):
            nv = (qrow + 1) // m
            idx[r, :nv] = e0 + np.arange(nv)
        outs.append(orc.attend_rows(q, shift, E, m, rows, "csa", idx=idx, win=kv,
                                    win_pos0=shift, sink=sink))
    assert np.allclose(outs[0], outs[1], atol=2e-6)


def test_layer_end_to_end_vs_bruteforce(orc):
    """compress -> bf16 indexer -> top-k -> attention, oracle vs brute force."""
    rng = np.random.default_rng(18)
    n, H, H_I, m = 64, 4, 2, 4
    q = _rand_bf16(rng, (n, H, 128))
    kv = _rand_bf16(rng, (n, 128), 0.3)
    ik = _rand_bf16(rng, (n, 64), 0.3)
    qI = _rand_bf16(rng, (n, H_I, 64), 0.3)
    w = rng.standard_normal((n, H_I)).astype(np.float32)
    beta = rng.standard_normal(8).astype(np.float32)
    sink = rng.standard_normal(H).astype(np.float32)
    ent, kid = orc.compress(kv, beta, m, 1, ik=ik)
    C, Ek = bf.compress(kv, beta, m, 1, ik_bits=ik)
    rows = np.arange(n, dtype=np.int32)
    qd = bf.bf16_bits_to_f64(qI).astype(np.float32)
    for k in [1, 3, 16]:
        idx = orc.index_topk_rows(qd, w, kid, m, 0, rows, k)
        sc = bf.index_scores(qd.astype(np.float64), w.astype(np.float64), Ek)
        nv = (np.arange(n) + 1) // m
        ref_idx = bf.topk_rows(sc, nv, k)
        # scores from fp32 vs fp64 pooling: equal unless within rounding of a tie
        for t in range(n):
            if not np.array_equal(idx[t], ref_idx[t]):
                a = set(idx[t][idx[t] >= 0]) ^ set(ref_idx[t][ref_idx[t] >= 0])
                kth = np.sort(sc[t, :nv[t]])[::-1][min(k, nv[t]) - 1]
                assert all(abs(sc[t, s] - kth) < 1e-6 for s in a)
        got = orc.attend_rows(q, 0, ent.astype(np.float64), m, rows, "csa", idx=idx, win=kv, sink=sink)
        ref = bf.attend(q, 0, C, m, "csa", idx=idx, win_bits=kv, sink=sink)
        assert np.allclose(got, ref, atol=1e-6)
