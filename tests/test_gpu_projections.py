"""GPU parity of the projections around the attention path (csa_project_in,
csa_project_qidx, csa_project_out) against oracle/projections.py, through
the C ABI.  Marked gpu.

Bounds (derived from the arithmetic; the kernel sums exact bf16 x bf16
products in fp32 over K terms, the oracle in fp64):
  * fp32 outputs:  |gpu - ref| <= K * 2^-23 * S + 2^-24 |ref|
  * bf16 outputs:  |gpu - ref| <= K * 2^-23 * S + 2^-8  |ref|
    (S = sum_k |x_k w_k|, the condition of the dot product; the 2^-8 covers
    the two roundings to bf16 of nearby fp32 values).
  * MXFP4 indexer query: the encoding is an integer decision taken in the
    kernel's fp32, so the codes and scales must equal the oracle encoder's
    output on the kernel's own fp32 values bit for bit, and those values
    obey the fp32 bound above.
"""
import numpy as np
import pytest
import torch

import long_context_attention_21_amd as L
from long_context_attention_21_amd import synth

from _helpers import dev, host, host_bits

pytestmark = pytest.mark.gpu


def _w(rng, shape, scale):
    return synth.to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _cond(x_bits, w_bits):
    return np.abs(_f64(x_bits)) @ np.abs(_f64(w_bits)).T


def _check_bf16(got_bits, ref64, S, K, what):
    g = _f64(got_bits)
    lim = K * 2.0 ** -23 * S + 2.0 ** -8 * np.abs(ref64)
    bad = np.abs(g - ref64) > lim
    assert not bad.any(), "%s: %d of %d outside the bound, first at %s" % (
        what, int(bad.sum()), bad.size, np.argwhere(bad)[0])


def _check_f32(got, ref64, S, K, what):
    lim = K * 2.0 ** -23 * S + 2.0 ** -24 * np.abs(ref64)
    bad = np.abs(got.astype(np.float64) - ref64) > lim
    assert not bad.any(), "%s: %d of %d outside the bound" % (what, int(bad.sum()), bad.size)


# the e2m1 grid's rounding midpoints (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6)
_E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def _nibbles(codes):
    c = np.asarray(codes, np.uint8)
    return np.stack([c & 15, c >> 4], axis=-1).reshape(c.shape[0], -1)


def _check_qidx_codes(orc, codes, scales, qf, lat, lat_orc, w_up):
    """The kernel's MXFP4 indexer query against the oracle's, which starts
    from the oracle's own bf16 latent.  The kernel's fp32 q_I may sit at most
    delta from the oracle's exact value: the latent difference carried
    through w_up exactly, plus the fp32 accumulation bound and one fp32
    rounding.  Every code or scale that differs must then lie at a rounding
    boundary: the oracle's scaled value within delta of an e2m1 midpoint, or
    its block maximum within delta of a power of two (where the shared scale
    steps)."""
    from oracle import projections as P
    r = lat.shape[1]
    q_o = P.linear_f64(lat_orc, w_up)
    delta = (np.abs(_f64(lat) - _f64(lat_orc)) @ np.abs(_f64(w_up)).T
             + r * 2.0 ** -23 * _cond(lat, w_up) + 2.0 ** -23 * np.abs(q_o))
    far = np.abs(qf.astype(np.float64) - q_o) > delta
    assert not far.any(), "q_I: %d values farther from the oracle than the bound" % int(far.sum())
    co, so = orc.mxfp4_encode(q_o.astype(np.float32))
    M, n = q_o.shape
    nb = n // 32
    sk, so = np.asarray(scales).reshape(M, nb), so.reshape(M, nb)
    ck, co = _nibbles(codes), _nibbles(co)
    q_b, d_b = q_o.reshape(M, nb, 32), delta.reshape(M, nb, 32)
    amax, dmax = np.abs(q_b).max(axis=2), d_b.max(axis=2)
    # a block whose scale differs: its maximum sits within delta of 2^e
    for i, b in np.argwhere(sk != so):
        thr = 2.0 ** np.round(np.log2(amax[i, b]))
        assert abs(amax[i, b] - thr) <= dmax[i, b], "q_I row %d block %d: scale differs away from a boundary" % (i, b)
    # a code that differs under the same scale: the scaled value sits within delta of a midpoint
    same_scale = np.repeat(sk == so, 32, axis=1)
    bad = np.argwhere((ck != co) & same_scale)
    for i, e in bad:
        unit = 2.0 ** (int(so[i, e // 32]) - 127)
        dist = np.abs(np.abs(q_o[i, e]) / unit - _E2M1_MID).min()
        assert dist <= delta[i, e] / unit, "q_I row %d elem %d: code differs away from a boundary" % (i, e)
    return int(bad.shape[0]) + int((sk != so).sum())


def _layer_weights(rng, d, H, H_I, r):
    return dict(w_q=_w(rng, (H * 128, d), d ** -0.5), w_kv=_w(rng, (128, d), d ** -0.5),
                w_ik=_w(rng, (64, d), d ** -0.5), w_lat=_w(rng, (r, d), d ** -0.5),
                w_w=_w(rng, (H_I, d), d ** -0.5), w_z=_w(rng, (2, d), d ** -0.5),
                w_up=_w(rng, (H_I * 64, r), r ** -0.5))


def _run_in(x, W, n_qidx=None):
    names = ("w_q", "w_kv", "w_ik", "w_lat", "w_w", "w_z")
    w_in = np.concatenate([W[k] for k in names], axis=0)
    widths = tuple(W[k].shape[0] for k in names)
    out = L.csa_project_in(dev(x), dev(w_in), widths, w_up=dev(W["w_up"]),
                           n_qidx=W["w_up"].shape[0] if n_qidx is None else n_qidx)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("M,d,H,H_I,r", [
    (300, 256, 4, 8, 32),     # ragged rows, 6 column tiles with a ragged last one, 8 K steps
    (129, 32, 2, 4, 16),      # one K step (less than the ring), one ragged row tile
    (1, 96, 1, 2, 64),        # a single row, 3 K steps
    (1100, 256, 4, 8, 32),    # 256 x 256 tiles: ragged row and column tiles
])
def test_project_in_matches_oracle(orc, M, d, H, H_I, r):
    from oracle import projections as P
    print("project_in case M=%d d=%d H=%d H_I=%d r=%d" % (M, d, H, H_I, r), flush=True)
    rng = np.random.default_rng(7000 + M)
    x = _w(rng, (M, d), 1.0)
    W = _layer_weights(rng, d, H, H_I, r)
    out = _run_in(x, W)
    ref = P.project_in(x, W["w_q"], W["w_kv"], W["w_ik"], W["w_lat"], W["w_w"], W["w_up"], w_z=W["w_z"])
    for name, wname in (("q", "w_q"), ("kv", "w_kv"), ("ik", "w_ik"), ("lat", "w_lat")):
        _check_bf16(host_bits(out[name]), P.linear_f64(x, W[wname]), _cond(x, W[wname]), d, name)
    _check_f32(host(out["w"]), P.linear_f64(x, W["w_w"]), _cond(x, W["w_w"]), d, "w_I")
    _check_f32(host(out["z"]), ref["z"].astype(np.float64), _cond(x, W["w_z"]), d, "z")
    # the indexer query of the kernel's own latent
    lat = host_bits(out["lat"])
    codes, scales, qf = L.csa_project_qidx(out["lat"], dev(W["w_up"]), with_f32=True)
    torch.cuda.synchronize()
    qf = host(qf)
    _check_f32(qf, P.linear_f64(lat, W["w_up"]), _cond(lat, W["w_up"]), r, "q_I fp32")
    rc, rs = orc.mxfp4_encode(qf)
    assert np.array_equal(host(codes), rc) and np.array_equal(host(scales), rs)
    assert np.array_equal(host(out["qidx"]), rc) and np.array_equal(host(out["qidx_scale"]), rs)
    # end to end against the oracle's codes (its latent may differ by an ulp)
    _check_qidx_codes(orc, host(out["qidx"]), host(out["qidx_scale"]), qf, lat, ref["lat"], W["w_up"])


@pytest.mark.parametrize("r", [16, 32, 64])
def test_project_qidx_on_oracle_latent(orc, r):
    """Given the oracle's bf16 latent, the kernel's fp32 q_I stays within the
    fp32 bound and its MXFP4 encoding is the oracle encoder's, bit for bit;
    zero rows give zero codes and a zero scale byte."""
    from oracle import projections as P
    rng = np.random.default_rng(80 + r)
    M, n_qidx = 77, 512
    lat = _w(rng, (M, r), 1.0)
    lat[5] = 0                       # an all-zero row
    lat[6, : r // 2] = 0
    w_up = _w(rng, (n_qidx, r), r ** -0.5)
    codes, scales, qf = L.csa_project_qidx(dev(lat), dev(w_up), with_f32=True)
    torch.cuda.synchronize()
    qf = host(qf)
    _check_f32(qf, P.linear_f64(lat, w_up), _cond(lat, w_up), r, "q_I fp32")
    rc, rs = orc.mxfp4_encode(qf)
    assert np.array_equal(host(codes), rc) and np.array_equal(host(scales), rs)
    assert not host(codes)[5].any() and not host(scales)[5].any()


@pytest.mark.parametrize("M,H,G,d", [
    (300, 8, 4, 256),     # 4 groups of 2 heads, 64 output columns per group
    (130, 4, 1, 384),     # G = 1: a dense projection, 3 column tiles
    (65, 16, 16, 2048),   # one head per group, 128 columns per group
    (3, 8, 2, 512),
    (1030, 16, 8, 2048),  # 256 x 256 tiles over 8 groups, ragged rows
    (1500, 4, 1, 768),    # 256 x 256 tiles, dense, 3 column tiles
])
def test_project_out_matches_oracle(M, H, G, d):
    from oracle import projections as P
    print("project_out case M=%d H=%d G=%d d=%d" % (M, H, G, d), flush=True)
    rng = np.random.default_rng(9000 + M)
    KG = H // G * 128
    o = _w(rng, (M, H * 128), 1.0)
    w_o = _w(rng, (d, KG), KG ** -0.5)
    y = L.csa_project_out(dev(o).view(M, H, 128), dev(w_o), G)
    torch.cuda.synchronize()
    _, ref = P.project_out(o, w_o, G)
    dg = d // G
    S = np.concatenate([_cond(o[:, j * KG:(j + 1) * KG], w_o[j * dg:(j + 1) * dg]) for j in range(G)], axis=1)
    _check_bf16(host_bits(y), ref, S, KG, "y")


def test_project_out_groups_do_not_mix():
    """Zeroing group j's head outputs zeroes exactly output columns
    [j*d/G, (j+1)*d/G) and leaves every other column bit-identical."""
    rng = np.random.default_rng(11)
    M, H, G, d = 200, 8, 4, 512
    KG, dg = H // G * 128, d // G
    o = _w(rng, (M, H * 128), 1.0)
    w_o = _w(rng, (d, KG), KG ** -0.5)
    y0 = host_bits(L.csa_project_out(dev(o).view(M, H, 128), dev(w_o), G))
    o[:, KG:2 * KG] = 0
    y1 = host_bits(L.csa_project_out(dev(o).view(M, H, 128), dev(w_o), G))
    assert not y1[:, dg:2 * dg].any()
    keep = np.r_[0:dg, 2 * dg:d]
    assert np.array_equal(y0[:, keep], y1[:, keep])


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_projections_full_size_sampled_rows(orc):
    """The chunk shape of the 1M-context prefill (8192 tokens, hidden 4096,
    64 query heads, 8 indexer heads of rank-32 latent, 8 output groups), in
    the launch configuration the benchmark times; rows sampled (first, last
    and ragged-tile rows included)."""
    from oracle import projections as P
    rng = np.random.default_rng(4)
    M, d, H, H_I, r, G = 8192, 4096, 64, 8, 32, 8
    print("project full size M=%d d=%d" % (M, d), flush=True)
    x = synth.normal_bf16(rng, (M, d), 1.0).reshape(M, d)
    W = _layer_weights(rng, d, H, H_I, r)
    out = _run_in(x, W)
    rows = np.unique(np.r_[0, 1, 127, 128, M - 1, rng.choice(M, 27, replace=False)])
    xs = x[rows]
    for name, wname in (("q", "w_q"), ("kv", "w_kv"), ("ik", "w_ik"), ("lat", "w_lat")):
        _check_bf16(host_bits(out[name])[rows], P.linear_f64(xs, W[wname]), _cond(xs, W[wname]), d, name)
    _check_f32(host(out["w"])[rows], P.linear_f64(xs, W["w_w"]), _cond(xs, W["w_w"]), d, "w_I")
    _check_f32(host(out["z"])[rows], P.linear_f64(xs, W["w_z"]), _cond(xs, W["w_z"]), d, "z")
    lat = host_bits(out["lat"])[rows]
    _, _, qf = L.csa_project_qidx(out["lat"], dev(W["w_up"]), with_f32=True)
    torch.cuda.synchronize()
    lat_orc = P.project_in(xs, W["w_q"][:1], W["w_kv"][:1], W["w_ik"][:1], W["w_lat"], W["w_w"][:1],
                           W["w_up"])["lat"]
    _check_qidx_codes(orc, host(out["qidx"])[rows], host(out["qidx_scale"])[rows], host(qf)[rows], lat, lat_orc,
                      W["w_up"])
    KG = H // G * 128
    o = synth.normal_bf16(rng, (M, H * 128), 1.0).reshape(M, H * 128)
    w_o = _w(rng, (d, KG), KG ** -0.5)
    y = host_bits(L.csa_project_out(dev(o).view(M, H, 128), dev(w_o), G))[rows]
    _, ref = P.project_out(o[rows], w_o, G)
    dg = d // G
    os_ = o[rows]
    S = np.concatenate([_cond(os_[:, j * KG:(j + 1) * KG], w_o[j * dg:(j + 1) * dg]) for j in range(G)], axis=1)
    _check_bf16(y, ref, S, KG, "y")


def test_csa_layer_forward_from_hidden_state(orc):
    """One CSA attention layer from the hidden state: csa_project_in ->
    csa_compress (kv, indexer keys, the projected compression logits z) ->
    csa_index_topk (the projected MXFP4 indexer query and head weights) ->
    csa_attend (window = the projected kv rows, sink) -> csa_project_out.
    Each stage is checked against the oracle given the GPU's bytes of the
    stage before: compression and the MXFP4 top-k bit-exactly, attention to
    the output tolerance, the projections to the bounds above."""
    from oracle import projections as P
    from _helpers import assert_close, canon_idx, oracle_compress_store
    rng = np.random.default_rng(21)
    M, d, H, H_I, r, G, m, k = 512, 256, 8, 8, 32, 4, 4, 32
    print("layer forward M=%d d=%d H=%d" % (M, d, H), flush=True)
    x = _w(rng, (M, d), 1.0)
    W = _layer_weights(rng, d, H, H_I, r)
    beta = rng.standard_normal(2 * m).astype(np.float32)
    sink = rng.standard_normal(H).astype(np.float32)
    KG = H // G * 128
    w_o = _w(rng, (d, KG), KG ** -0.5)
    out = _run_in(x, W)
    q = out["q"].view(1, M, H, 128)
    comp = L.csa_compress(out["kv"].view(1, M, 128), dev(beta), m, 1, ik=out["ik"].view(1, M, 64),
                          z=out["z"].view(1, M, 2), kidx_fmt="mxfp4")
    idx = L.csa_index_topk(out["qidx"].view(1, M, H_I, 32), out["w"].view(1, M, H_I), comp["kidx"], k, m,
                           fmt="mxfp4", qidx_scale=out["qidx_scale"].view(1, M, H_I, 2),
                           kidx_scale=comp["kidx_scale"])
    o = L.csa_attend(q, comp["entries"], idx, m=m, win_kv=out["kv"].view(1, M, 128), sink=dev(sink))
    y = L.csa_project_out(o, dev(w_o), G)
    torch.cuda.synchronize()
    # projections
    for name, wname in (("q", "w_q"), ("kv", "w_kv"), ("ik", "w_ik")):
        _check_bf16(host_bits(out[name]), P.linear_f64(x, W[wname]), _cond(x, W[wname]), d, name)
    _check_f32(host(out["z"]), P.linear_f64(x, W["w_z"]), _cond(x, W["w_z"]), d, "z")
    # compression of the projected rows
    kv, ik, z = host_bits(out["kv"]), host_bits(out["ik"]), host(out["z"])
    ref = oracle_compress_store(orc, kv, beta, m, 1, ik=ik, z=z, kidx_fmt="mxfp4")
    assert np.array_equal(host_bits(comp["entries"])[0], ref["entries"])
    assert np.array_equal(host(comp["kidx"])[0], ref["kidx"])
    assert np.array_equal(host(comp["kidx_scale"])[0], ref["kidx_scale"])
    # top-k from the projected MXFP4 query
    qdec = orc.mxfp4_decode(host(out["qidx"]), host(out["qidx_scale"])).reshape(M, H_I, 64)
    rows = np.arange(M, dtype=np.int32)
    ref_idx = orc.index_topk_rows(qdec, host(out["w"]), ref["kidx_dec"], m, 0, rows, k)
    got_idx = host(idx)[0]
    assert np.array_equal(canon_idx(got_idx), ref_idx)
    # attention
    ref_o = orc.attend_rows(host_bits(out["q"]).reshape(M, H, 128), 0, ref["entries_f64"], m, rows, "csa",
                            idx=ref_idx, win=kv, sink=sink)
    assert_close(host_bits(o)[0], ref_o, "layer attention")
    # output projection of the GPU's attention output
    o_bits = host_bits(o).reshape(M, H * 128)
    _, ref_y = P.project_out(o_bits, w_o, G)
    dg = d // G
    S = np.concatenate([_cond(o_bits[:, j * KG:(j + 1) * KG], w_o[j * dg:(j + 1) * dg]) for j in range(G)], axis=1)
    _check_bf16(host_bits(y), ref_y, S, KG, "y")
