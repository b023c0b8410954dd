"""Pins of the projection oracle (oracle/projections.py) against facts that
do not come from its own formula: brute-force sums on tiny inputs, exact
scaling, the identity map, the block-diagonal structure of the grouped
output projection and its invariance under a consistent permutation of the
heads inside a group, and the MXFP4 encoding of a selected latent.  CPU
only."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import projections as P


def _bits(rng, shape, scale=1.0):
    return oracle.bf16_from_f32((rng.standard_normal(shape) * scale).astype(np.float32))


def _frac(b):
    return [[Fraction(float(v)) for v in row] for row in oracle.bf16_to_f64(b)]


def test_linear_matches_exact_brute_force():
    """Each output is the exactly summed product, rounded to fp32 then bf16."""
    rng = np.random.default_rng(0)
    x, w = _bits(rng, (3, 7)), _bits(rng, (5, 7))
    xf, wf = _frac(x), _frac(w)
    exact = np.array([[float(sum(a * b for a, b in zip(xr, wr))) for wr in wf] for xr in xf])
    got = P.linear_f64(x, w)
    assert np.allclose(got, exact, rtol=1e-15, atol=0)
    want = oracle.bf16_from_f32(exact.astype(np.float32))
    assert np.array_equal(P._bf16(got), want)


def test_linear_scales_exactly():
    rng = np.random.default_rng(1)
    x, w = _bits(rng, (4, 64)), _bits(rng, (6, 64))
    x2 = oracle.bf16_from_f32(2.0 * oracle.bf16_to_f64(x).astype(np.float32))
    assert np.array_equal(P.linear_f64(x2, w), 2.0 * P.linear_f64(x, w))


def test_identity_projection_returns_the_input():
    rng = np.random.default_rng(2)
    d = 32
    x = _bits(rng, (5, d))
    eye = oracle.bf16_from_f32(np.eye(d, dtype=np.float32))
    w_up = oracle.bf16_from_f32(np.zeros((2 * 64, 4), np.float32))   # H_I = 2, r = 4
    r = P.project_in(x, eye, eye[:16], eye[:8], eye[:4], eye[:2], w_up, w_z=eye[5:7])
    assert np.array_equal(r["q"], x)
    assert np.array_equal(r["kv"], x[:, :16])
    assert np.array_equal(r["ik"], x[:, :8])
    assert np.array_equal(r["lat"], x[:, :4])
    assert np.array_equal(r["w_I"], oracle.bf16_to_f64(x[:, :2]).astype(np.float32))
    assert np.array_equal(r["z"], oracle.bf16_to_f64(x[:, 5:7]).astype(np.float32))
    assert not r["q_I_f32"].any() and not r["q_I_codes"].any() and not r["q_I_scales"].any()


def test_indexer_query_is_the_mxfp4_encoding_of_the_projected_latent():
    """With W_up rows selecting latent components, q_I is the latent itself,
    and its codes are the pinned encoder's codes of those values."""
    rng = np.random.default_rng(3)
    d, r, H_I = 16, 8, 2
    x = _bits(rng, (6, d))
    w_lat = _bits(rng, (r, d), 0.5)
    sel = np.zeros((H_I * 64, r), np.float32)
    for i in range(H_I * 64):
        sel[i, i % r] = 1.0
    zero = oracle.bf16_from_f32(np.zeros((1, d), np.float32))
    res = P.project_in(x, zero, zero, zero, w_lat, zero, oracle.bf16_from_f32(sel))
    lat = oracle.bf16_to_f64(res["lat"]).astype(np.float32)
    want = lat[:, np.arange(H_I * 64) % r]
    assert np.array_equal(res["q_I_f32"], want)
    codes, scales = oracle.mxfp4_encode(want)
    assert np.array_equal(res["q_I_codes"], codes)
    assert np.array_equal(res["q_I_scales"], scales)


def _grouped_inputs(seed, M=5, H=8, G=4, d=32):
    rng = np.random.default_rng(seed)
    o = _bits(rng, (M, H * 128))
    w = _bits(rng, (d, H // G * 128), 1 / 16)
    return o, w, G


def test_grouped_projection_is_block_diagonal():
    o, w, G = _grouped_inputs(4)
    y0, y0f = P.project_out(o, w, G)
    d = w.shape[0]
    dg, KG = d // G, w.shape[1]
    for j in range(G):
        o2 = o.copy()
        o2[:, j * KG:(j + 1) * KG] = 0           # +0 bits
        y, yf = P.project_out(o2, w, G)
        assert not yf[:, j * dg:(j + 1) * dg].any()
        keep = np.ones(d, bool)
        keep[j * dg:(j + 1) * dg] = False
        assert np.array_equal(yf[:, keep], y0f[:, keep])


def test_grouped_projection_with_one_group_is_dense():
    o, w, _ = _grouped_inputs(5, H=2, G=1)
    y, yf = P.project_out(o, w, 1)
    assert np.array_equal(yf, P.linear_f64(o, w))


def test_grouped_projection_invariant_under_head_permutation_within_a_group():
    o, w, G = _grouped_inputs(6)
    KG = w.shape[1]
    hpg = KG // 128
    perm = np.random.default_rng(7).permutation(hpg)
    o2, w2 = o.copy(), w.copy()
    for j in range(G):
        blk = o[:, j * KG:(j + 1) * KG].reshape(o.shape[0], hpg, 128)
        o2[:, j * KG:(j + 1) * KG] = blk[:, perm].reshape(o.shape[0], KG)
    w2[:] = w.reshape(w.shape[0], hpg, 128)[:, perm].reshape(w.shape)
    a, af = P.project_out(o, w, G)
    b, bf = P.project_out(o2, w2, G)
    assert np.allclose(af, bf, rtol=1e-12, atol=1e-12)
