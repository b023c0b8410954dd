"""Parity at the full workload sizes, in the launch configuration bench.py
times (the same workload classes build the inputs and run the step).

Compression and the stored caches are checked bit-exactly over every row.
Top-k (bit-exact: MXFP4 scores are exact) and attention (max-abs 2e-2 /
mean-rel 5e-3 against the fp64 oracle) are checked on every query row of the
HCA layer at 32K and every sequence of the decode step, and on at least 1024
stratified rows of the 128K prefill and the 1M chunk: all of the first 256
rows, then rows spread uniformly to the end, plus the ragged and boundary
rows.
"""
import numpy as np
import pytest

from _helpers import assert_close, canon_idx

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _rows(n, count, seed, extra=()):
    rng = np.random.default_rng(seed)
    r = set(int(x) for x in rng.choice(n, size=min(count, n), replace=False))
    r.update(int(x) for x in extra if 0 <= x < n)
    return np.array(sorted(r), np.int32)


def _stratified(n, extra=()):
    """All of the first 256 rows, 768 rows spread uniformly over the rest,
    and the given rows: at least 1024."""
    r = set(range(min(256, n)))
    r.update(int(x) for x in np.linspace(256, n - 1, 768).round().astype(np.int64))
    r.update(int(x) for x in extra if 0 <= x < n)
    return np.array(sorted(r), np.int32)


@pytest.mark.timeout(600)
def test_config2_hca_full(orc):
    import bench
    wl = bench.HcaLayer(2)
    wl.step()
    torch.cuda.synchronize()
    c = wl.c
    ent, _ = orc.compress(c["kv"][0], c["beta"], wl.m, 0)
    e_bits = orc.bf16_from_f32(ent)
    assert np.array_equal(_bits(wl.bufs["entries"])[0], e_bits)
    # every query row, in blocks of 4096 (the error measures are taken over
    # each block)
    got = _bits(wl.out)[0]
    E = orc.bf16_to_f64(e_bits)
    for r0 in range(0, wl.n, 4096):
        rows = np.arange(r0, min(wl.n, r0 + 4096), dtype=np.int32)
        ref = orc.attend_rows(c["q"][0], 0, E, wl.m, rows, "hca", win=c["kv"][0], sink=c["sink"])
        assert_close(got[rows], ref, "config 2 hca_attend rows %d.." % r0)


@pytest.mark.timeout(600)
def test_config3_csa_full(orc):
    import bench
    wl = bench.CsaLayer(3)
    wl.fallbacks.zero_()
    wl.step()
    # rows whose k-th score falls on the point mass of exact zeros (every head
    # product <= 0 under mostly negative head weights) may take the exact
    # path: allow at most 8 work-groups (65,536 work-groups of 2 rows here)
    nfb = int(wl.fallbacks.item())
    assert nfb <= 8, "%d indexer work-groups took the exact streaming path" % nfb
    torch.cuda.synchronize()
    c = wl.c
    ent, kid = orc.compress(c["kv"][0], c["beta"], 4, 1, ik=c["ik"][0])
    e_bits = orc.bf16_from_f32(ent)
    kc, ks = orc.mxfp4_encode(kid)
    assert np.array_equal(_bits(wl.bufs["entries"])[0], e_bits)
    assert np.array_equal(wl.bufs["kidx"].cpu().numpy()[0], kc)
    assert np.array_equal(wl.bufs["kidx_scale"].cpu().numpy()[0], ks)
    # stratified rows plus those around n_vis = k (8192), the 2- to 4-token
    # boundary and the end
    rows = _stratified(wl.n, extra=(8190, 8191, 8192, 8195, 65536, wl.n - 4, wl.n - 1))
    assert rows.size >= 1024
    qc, qs = orc.mxfp4_encode(orc.bf16_to_f64(c["q_I"][0]).astype(np.float32))
    ref_idx = orc.index_topk_rows(orc.mxfp4_decode(qc, qs), c["w_I"][0], orc.mxfp4_decode(kc, ks), 4, 0,
                                  rows, wl.k)
    got_idx = wl.idx.cpu().numpy()[0][rows]
    bad = np.nonzero(~np.all(canon_idx(got_idx) == ref_idx, axis=1))[0]
    assert bad.size == 0, "config 3 top-k rows %s differ" % rows[bad[:5]]
    ref = orc.attend_rows(c["q"][0], 0, orc.bf16_to_f64(e_bits), 4, rows, "csa", idx=ref_idx, win=c["kv"][0],
                          sink=c["sink"])
    assert_close(_bits(wl.out)[0][rows], ref, "config 3 csa_attend")
    # the step pipelines the indexer and the attention over token chunks on
    # two streams (csa_index_attend): the calls in turn give the same bytes
    assert wl.chunks > 1
    piped_idx, piped_out = wl.idx.cpu().numpy().copy(), _bits(wl.out).copy()
    wl.idx.zero_()
    wl.out.zero_()
    wl.step(serial=True)
    torch.cuda.synchronize()
    assert np.array_equal(wl.idx.cpu().numpy(), piped_idx), "pipelined top-k differs from the calls in turn"
    assert np.array_equal(_bits(wl.out), piped_out), "pipelined attention differs from the calls in turn"


@pytest.mark.timeout(1100)
def test_config4_decode_full(orc):
    """Every one of the 64 sequences: the caches the step reads against the
    oracle's encoders of the same draws (bit-exact), the top-k set
    (bit-exact), the attention output; and the whole step run twice,
    bit-identical (the split indexer appends candidates in atomic order)."""
    import bench
    from long_context_attention_21_amd import synth
    wl = bench.DecodeLayer(4)
    wl.fallbacks.zero_()
    wl.step()
    assert int(wl.fallbacks.item()) == 0, "indexer took the exact streaming path"
    torch.cuda.synchronize()
    first_idx, first_out = wl.idx.cpu().numpy().copy(), _bits(wl.out).copy()
    wl.step()
    torch.cuda.synchronize()
    assert np.array_equal(wl.idx.cpu().numpy(), first_idx), "top-k differs run to run"
    assert np.array_equal(_bits(wl.out), first_out), "attention differs run to run"
    c = wl.c
    t = c["q_pos0"]
    q = _bits(wl.q)
    qI = _bits(wl.qI)
    w = wl.w.cpu().numpy()
    sink = wl.sink.cpu().numpy()
    got_idx = wl.idx.cpu().numpy()
    got_out = _bits(wl.out)
    draws = synth.config(4)  # the same seeded draws, in the same order
    for b in range(wl.B):
        print("config 4 sequence %d" % b, flush=True)
        ent, ik, swa = draws["seq"](b)
        codes, rope, scale = wl.codes[b].cpu().numpy(), _bits(wl.rope[b]), wl.scale[b].cpu().numpy()
        # the stored caches are csa_compress with one slot per entry (m = 1,
        # no rotation): the oracle's compressor, then its FP8 / MXFP4 stores
        e1, k1 = orc.compress(synth.to_bf16_bits(ent), np.zeros(1, np.float32), 1, 0,
                              ik=synth.to_bf16_bits(ik), rope_dims=0)
        rc, rr, rs = orc.store_entries_fp8(e1)
        for name, g_, r_ in (("codes", codes, rc), ("rope", rope, rr), ("scale", scale, rs)):
            bad = np.argwhere(g_ != r_)
            assert bad.size == 0, "sequence %d: %d %s differ, first at %s: gpu %s oracle %s" % (
                b, len(bad), name, bad[:4].tolist(), g_[tuple(bad[0])], r_[tuple(bad[0])])
        kc, ks = orc.mxfp4_encode(k1)
        assert np.array_equal(wl.kc[b].cpu().numpy(), kc) and np.array_equal(wl.ks[b].cpu().numpy(), ks), b
        assert np.array_equal(_bits(wl.swa[b]), swa), b
        kdec = orc.mxfp4_decode(kc, ks)
        E = orc.load_entries_fp8(rc, rr, rs)
        qc, qs = orc.mxfp4_encode(orc.bf16_to_f64(qI[b]).astype(np.float32))
        rows = np.zeros(1, np.int32)
        ref_idx = orc.index_topk_rows(orc.mxfp4_decode(qc, qs), w[b], kdec, 4, t, rows, wl.k)
        assert np.array_equal(canon_idx(got_idx[b]), ref_idx), "config 4 top-k of sequence %d differs" % b
        ref = orc.attend_rows(q[b], t, E, 4, rows, "csa", idx=ref_idx, win=_bits(wl.swa[b]),
                              win_pos0=c["win_pos0"], sink=sink)
        assert_close(got_out[b], ref, "config 4 csa_attend (sequence %d)" % b)


@pytest.mark.timeout(600)
def test_config4_decode_full_v41_layout(orc):
    """Config 4 in the V4.1 layout the benchmark times with --entry-fmt
    nvfp4: NVFP4 entries stored by csa_compress and the FP8 window ring
    written by csa_cache_append; sampled sequences against the oracle, the
    stored window bytes against the oracle's FP8 window rule."""
    import bench
    bench.DecodeLayer.entry_fmt = "nvfp4"
    try:
        wl = bench.DecodeLayer(4)
    finally:
        bench.DecodeLayer.entry_fmt = "fp8"
    wl.step()
    torch.cuda.synchronize()
    c = wl.c
    t = c["q_pos0"]
    q = _bits(wl.q)
    sink = wl.sink.cpu().numpy()
    got_idx = wl.idx.cpu().numpy()
    got_out = _bits(wl.out)
    j0 = c["win_pos0"]
    s0 = j0 - wl.win8_pos0
    for b in range(wl.B):
        codes8, sc8 = wl.win8[b].cpu().numpy(), wl.win8_scale[b].cpu().numpy()
        ref_c, ref_s = orc.store_window_fp8(_bits(wl.swa[b]), j0)
        assert np.array_equal(codes8[s0:s0 + c["n_win"]], ref_c)
        assert np.array_equal(sc8[s0:s0 + c["n_win"]], ref_s)
        E = orc.load_entries_nvfp4(wl.codes[b].cpu().numpy(), wl.scale[b].cpu().numpy())
        rows = np.zeros(1, np.int32)
        idx = got_idx[b]  # the top-k itself is checked bit-exactly in the FP8 layout test
        ref = orc.attend_rows(q[b], t, E, 4, rows, "csa", idx=idx, win_post=orc.load_window_fp8(codes8, sc8),
                              win_pos0=wl.win8_pos0, sink=sink)
        assert_close(got_out[b], ref, "config 4 V4.1 layout csa_attend (sequence %d)" % b)


@pytest.mark.timeout(600)
def test_config5_pair_full(orc):
    import bench
    wl = bench.PairLayer(5)
    wl.fallbacks.zero_()
    wl.step()
    # a few query rows whose head weights are (nearly) all negative have their
    # k-th score on the point mass of exact zeros (every head's dot product
    # <= 0): the cut then keeps more than a wave region holds and those work
    # groups take the exact path (2,048 work-groups of 4 rows here; 3 seen)
    nfb = int(wl.fallbacks.item())
    assert nfb <= 8, "%d indexer work-groups took the exact streaming path" % nfb
    torch.cuda.synchronize()
    cs, hs = wl.c["csa"], wl.c["hca"]
    P, n = wl.P, wl.n
    # the chunk's new entries (state of the previous block given)
    ent_new, kid_new = orc.compress(cs["kv_new"], cs["beta"], 4, 1, pos0=P, ik=cs["ik_new"],
                                    prev_kv=cs["state_kv"][124:], prev_ik=cs["state_ik"])
    e_new = orc.bf16_from_f32(ent_new)
    kn, ksn = orc.mxfp4_encode(kid_new)
    assert np.array_equal(_bits(wl.c_ent)[0][wl.Nc0:], e_new)
    assert np.array_equal(wl.c_kc.cpu().numpy()[0][wl.Nc0:], kn)
    assert np.array_equal(wl.c_ks.cpu().numpy()[0][wl.Nc0:], ksn)
    hent_new, _ = orc.compress(hs["kv_new"], hs["beta"], 128, 0, pos0=P)
    h_new = orc.bf16_from_f32(hent_new)
    assert np.array_equal(_bits(wl.h_ent)[0][wl.Nh0:], h_new)
    # the given caches as the library stored them
    kdec = orc.mxfp4_decode(wl.c_kc.cpu().numpy()[0], wl.c_ks.cpu().numpy()[0])
    E = orc.bf16_to_f64(_bits(wl.c_ent)[0])
    HE = orc.bf16_to_f64(_bits(wl.h_ent)[0])
    rows = _stratified(n, extra=(0, 1, 3, 4, 127, 128, n - 1))
    assert rows.size >= 1024
    qc, qs = orc.mxfp4_encode(orc.bf16_to_f64(cs["q_I"]).astype(np.float32))
    ref_idx = orc.index_topk_rows(orc.mxfp4_decode(qc, qs), cs["w_I"], kdec, 4, P, rows, wl.k)
    got_idx = wl.idx.cpu().numpy()[0][rows]
    bad = np.nonzero(~np.all(canon_idx(got_idx) == ref_idx, axis=1))[0]
    assert bad.size == 0, "config 5 top-k rows %s differ" % rows[bad[:5]]
    win_c = np.concatenate([cs["state_kv"], cs["kv_new"]])
    ref = orc.attend_rows(cs["q"], P, E, 4, rows, "csa", idx=ref_idx, win=win_c, win_pos0=P - 128,
                          sink=cs["sink"])
    assert_close(_bits(wl.c_out)[0][rows], ref, "config 5 csa_attend")
    win_h = np.concatenate([hs["state_kv"], hs["kv_new"]])
    ref = orc.attend_rows(hs["q"], P, HE, 128, rows, "hca", win=win_h, win_pos0=P - 128, sink=hs["sink"])
    assert_close(_bits(wl.h_out)[0][rows], ref, "config 5 hca_attend")
