"""GPU parity: each HIP entry point against the CPU oracle on the same
seeded inputs (per stage: both sides get exactly the same input bytes), at
sizes that span several tiles and a ragged tail.  Runs through the C ABI
via the Python binding.  Marked gpu."""
import numpy as np
import pytest
import torch

import long_context_attention_21_amd as L
from long_context_attention_21_amd import synth

from _helpers import (assert_close, bf16_f64, dev, host, host_bits, oracle_compress_store,
                      oracle_q_dec, topk_tie_ok, canon_idx, canonical_rows)

pytestmark = pytest.mark.gpu


def _bf16(rng, shape, scale):
    return synth.to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


# ------------------------------------------------------------------ compress --

@pytest.mark.parametrize("m,overlap,with_z,kfmt,efmt", [
    (4, 1, False, "mxfp4", "bf16"),
    (4, 1, True, "bf16", "bf16"),
    (4, 1, True, "mxfp4", "fp8"),
    (128, 0, False, None, "bf16"),
    (8, 0, True, "mxfp4", "fp8"),
    (4, 1, True, "mxfp4", "nvfp4"),
    (128, 0, False, None, "nvfp4"),
])
def test_compress_matches_oracle(orc, m, overlap, with_z, kfmt, efmt):
    rng = np.random.default_rng(100 + m)
    B, T = 2, 37 * m + 3
    print("compress case m=%d overlap=%d z=%s kfmt=%s efmt=%s" % (m, overlap, with_z, kfmt, efmt), flush=True)
    kv = _bf16(rng, (B, T, 128), 0.3)
    ik = _bf16(rng, (B, T, 64), 0.3) if kfmt else None
    z = rng.standard_normal((B, T, 2)).astype(np.float32) if with_z else None
    beta = rng.standard_normal(2 * m if overlap else m).astype(np.float32)
    out = L.csa_compress(dev(kv), dev(beta), m, overlap, ik=dev(ik) if ik is not None else None,
                         z=dev(z) if z is not None else None, entry_fmt=efmt,
                         kidx_fmt=kfmt or "mxfp4")
    torch.cuda.synchronize()
    for b in range(B):
        ref = oracle_compress_store(orc, kv[b], beta, m, overlap, ik=None if ik is None else ik[b],
                                    z=None if z is None else z[b], kidx_fmt=kfmt or "mxfp4",
                                    entry_fmt=efmt)
        if efmt == "bf16":
            assert np.array_equal(host_bits(out["entries"])[b], ref["entries"])
        elif efmt == "nvfp4":
            assert np.array_equal(host(out["entries"])[b], ref["entries"])
            assert np.array_equal(host(out["entry_scale"])[b], ref["entry_scale"])
        else:
            assert np.array_equal(host(out["entries"])[b], ref["entries"])
            assert np.array_equal(host_bits(out["entries_rope"])[b], ref["entries_rope"])
            assert np.array_equal(host(out["entry_scale"])[b], ref["entry_scale"])
        if kfmt == "mxfp4":
            assert np.array_equal(host(out["kidx"])[b], ref["kidx"])
            assert np.array_equal(host(out["kidx_scale"])[b], ref["kidx_scale"])
        elif kfmt == "bf16":
            assert np.array_equal(host_bits(out["kidx"])[b], ref["kidx"])


def test_compress_chunked_with_prev_rows(orc):
    """A chunk starting at pos0 > 0 with the previous block passed in gives
    the same entries as compressing the whole sequence."""
    rng = np.random.default_rng(7)
    T, m, p0 = 400, 4, 160
    kv = _bf16(rng, (1, T, 128), 0.3)
    ik = _bf16(rng, (1, T, 64), 0.3)
    z = rng.standard_normal((1, T, 2)).astype(np.float32)
    beta = rng.standard_normal(8).astype(np.float32)
    whole = L.csa_compress(dev(kv), dev(beta), m, 1, ik=dev(ik), z=dev(z))
    part = L.csa_compress(dev(kv[:, p0:]), dev(beta), m, 1, pos0=p0, ik=dev(ik[:, p0:]),
                          z=dev(z[:, p0:]), prev_kv=dev(kv[:, p0 - m:p0]),
                          prev_ik=dev(ik[:, p0 - m:p0]), prev_z=dev(z[:, p0 - m:p0]))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(part["entries"]), host_bits(whole["entries"])[:, p0 // m:])
    assert np.array_equal(host(part["kidx"]), host(whole["kidx"])[:, p0 // m:])
    ref = oracle_compress_store(orc, kv[0, p0:], beta, m, 1, ik=ik[0, p0:], z=z[0, p0:], pos0=p0,
                                prev_kv=kv[0, p0 - m:p0], prev_ik=ik[0, p0 - m:p0],
                                prev_z=z[0, p0 - m:p0])
    assert np.array_equal(host_bits(part["entries"])[0], ref["entries"])


# ------------------------------------------------------------------- indexer --

def _index_case(orc, rng, B, n, N, H_I, k, q_pos0, fmt, m=4, dup_rows=0, prequant=False,
                key_scale=1.0, fallback=False):
    q = _bf16(rng, (B, n, H_I, 64), 1 / 8)
    w = (rng.standard_normal((B, n, H_I)) / np.sqrt(H_I)).astype(np.float32)
    kf = (rng.standard_normal((B, N, 64)) * key_scale / 8).astype(np.float32)
    if dup_rows:
        kf = kf[:, rng.integers(0, dup_rows, N)]          # force exact score ties
    if fmt == "mxfp4":
        kc, ks = orc.mxfp4_encode(kf)
        kdec = orc.mxfp4_decode(kc, ks)
        kdev, ksdev = dev(kc), dev(ks)
    else:
        kc = orc.bf16_from_f32(kf)
        kdec = orc.bf16_to_f64(kc).astype(np.float32)
        kdev, ksdev = dev(kc), None
    qdec = oracle_q_dec(orc, q, fmt)
    fc = torch.zeros(1, dtype=torch.int32, device="cuda")
    if prequant:
        qc, qs = orc.mxfp4_encode(orc.bf16_to_f64(q).astype(np.float32))
        got = L.csa_index_topk(dev(qc), dev(w), kdev, k, m, q_pos0=q_pos0, fmt=fmt,
                               qidx_scale=dev(qs), kidx_scale=ksdev, fallback_count=fc)
    else:
        got = L.csa_index_topk(dev(q), dev(w), kdev, k, m, q_pos0=q_pos0, fmt=fmt, kidx_scale=ksdev,
                               fallback_count=fc)
    torch.cuda.synchronize()
    nfb = int(fc.item())
    # the sampled threshold leaves between k and 4096 candidates on untied
    # scores; the exact streaming path is for massive ties only
    if fallback is not None:
        assert (nfb > 0) == fallback, "%d work-groups took the exact streaming path" % nfb
    got = host(got)
    rows = np.arange(n, dtype=np.int32)
    # every row in the canonical order, then the -1 padding
    assert np.array_equal(got, canonical_rows(got)), "rows are not in the canonical order"
    for b in range(B):
        ref = orc.index_topk_rows(qdec[b], w[b], kdec[b], m, q_pos0, rows, k)
        if fmt == "mxfp4":
            # the oracle's rows are ascending: compare the sets
            bad = np.nonzero(~np.all(canon_idx(got[b]) == ref, axis=1))[0]
            assert bad.size == 0, "rows %s differ (first: gpu %s ref %s)" % (
                bad[:5], got[b][bad[0]][:8], ref[bad[0]][:8])
        else:
            nv = np.minimum(N, (q_pos0 + rows + 1) // m)
            scores = np.zeros((n, N), np.float32)
            for r in range(n):
                scores[r, :nv[r]] = orc.index_scores(qdec[b, r], w[b, r], kdec[b, :nv[r]])
            topk_tie_ok(got[b], ref, scores, nv, k)


@pytest.mark.parametrize("B,n,N,H_I,k,q_pos0,fmt,extra", [
    (2, 301, 75, 8, 16, 0, "mxfp4", {}),             # fast path + selection, ragged tail
    (1, 37, 20000, 8, 2048, 80000 - 37, "mxfp4", {}),  # several exact shrinks per token
    (1, 50, 3000, 8, 64, 12000, "mxfp4", {"dup_rows": 40, "fallback": None}),  # massive exact ties
    (1, 40, 20000, 8, 2048, 80000 - 40, "mxfp4", {"dup_rows": 3, "fallback": True}),  # ties overflow -> exact path
    (1, 41, 9000, 8, 2048, 36000 - 41, "mxfp4", {}),  # sampled threshold, stride 3
    (3, 1, 20000, 8, 2048, 80000, "mxfp4", {}),       # decode path, one token per sequence
    (1, 64, 2000, 8, 100, 8000, "mxfp4", {"prequant": True}),
    (1, 301, 75, 4, 16, 0, "bf16", {}),               # bf16 indexer, 4 heads
    (1, 40, 5000, 1, 300, 20000, "bf16", {}),
    # split path (few query rows over >= 65536 visible entries): partitions of
    # up to 262144 visible entries each keep their highest scores by their
    # own cut; longer rows take a sampled threshold per row first; then the
    # selection per row
    (1, 9, 70000, 8, 2048, 280000 - 9, "mxfp4", {}),     # long rows: 4-token work-groups
    (3, 1, 70000, 8, 512, 280000, "mxfp4", {}),          # ragged last partition
    (2, 4, 90000, 8, 2048, 280000 - 4, "mxfp4", {}),     # entries past the causal bound
    (1, 2, 70000, 8, 512, 280000, "mxfp4", {"dup_rows": 3, "fallback": True}),  # candidates overflow
    (2, 1, 66000, 4, 300, 264000, "bf16", {}),
    (2, 1, 300000, 8, 2048, 1200000, "mxfp4", {}),     # past 262144 entries: sampled threshold first
    (1, 3, 262144, 8, 2048, 1048576 - 3, "mxfp4", {}),  # 16 full partitions
])
def test_index_topk_matches_oracle(orc, B, n, N, H_I, k, q_pos0, fmt, extra):
    print("index case B=%d n=%d N=%d H_I=%d k=%d pos0=%d %s %s" % (B, n, N, H_I, k, q_pos0, fmt, extra),
          flush=True)
    _index_case(orc, np.random.default_rng(N + n), B, n, N, H_I, k, q_pos0, fmt, **extra)


# ----------------------------------------------------------------- attention --

def _with_offset(rng, shape, scale, offset):
    """bf16 N(0,1) * scale draws, plus `offset` on dim 0 (not rotated)."""
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    x[..., 0] += np.float32(offset)
    return synth.to_bf16_bits(x)


def _attend_case(orc, seed, B, n, H, q_pos0, m, mode, k=0, n_win=128, sink=True, q_scale=1.0,
                 efmt="bf16", kv_scale=None, sink_shift=0.0, check_rows=None, wfmt="bf16",
                 kv_offset=0.0, q_offset=0.0, sink_heads=None, forced_rerun=None):
    """One attention call against the oracle.  kv_offset / q_offset add a
    constant to dim 0 of every raw KV row / query row; sink_heads (a boolean
    mask over heads) applies sink_shift to those heads only.  forced_rerun
    "overflow" / "underflow" asserts from the inputs that every checked row
    sum leaves [2^-100, 2^100) against the kernel's first reference (the
    sink logit; 0 without a sink), so the max-only pass must run."""
    rng = np.random.default_rng(seed)
    T = q_pos0 + n
    kv_scale = kv_scale or 1 / np.sqrt(128)
    if kv_offset:
        kv = _with_offset(rng, (B, T, 128), kv_scale, kv_offset)
    else:
        kv = _bf16(rng, (B, T, 128), kv_scale)
    if q_offset:
        q = _with_offset(rng, (B, n, H, 128), q_scale / np.sqrt(128), q_offset)
    else:
        q = _bf16(rng, (B, n, H, 128), q_scale / np.sqrt(128))
    beta = rng.standard_normal(2 * m if mode == "csa" else m).astype(np.float32)
    sk = None
    if sink:
        sh = sink_shift if sink_heads is None else np.where(sink_heads, sink_shift, 0.0)
        sk = (rng.standard_normal(H) + sh).astype(np.float32)
    ents = [oracle_compress_store(orc, kv[b], beta, m, 1 if mode == "csa" else 0, entry_fmt=efmt)
            for b in range(B)]
    N = ents[0]["entries_f64"].shape[0]
    rows = np.arange(n, dtype=np.int32)
    idx = None
    if mode == "csa":
        idx = np.full((B, n, k), -1, np.int32)
        for b in range(B):
            for r in range(n):
                nv = min(N, (q_pos0 + r + 1) // m)
                c = min(k, nv)
                if c:
                    idx[b, r, :c] = np.sort(rng.choice(nv, size=c, replace=False))
    e_dev = dev(np.stack([e["entries"] for e in ents]))
    win = dev(kv) if n_win > 0 else None
    win8 = None
    if wfmt == "fp8":  # the FP8 window cache of the whole sequence, from the oracle
        win8 = [orc.store_window_fp8(kv[b], 0) for b in range(B)]
        win = dev(np.stack([w[0] for w in win8]))
    roped = None
    if wfmt == "roped":  # rows rotated once at their positions, from the oracle
        roped = np.stack([orc.rope_rows_bf16(kv[b], 0) for b in range(B)])
        win = dev(roped)
    if mode == "csa":
        kw = {}
        if efmt == "fp8":
            kw = dict(entries_rope=dev(np.stack([e["entries_rope"] for e in ents])),
                      entry_scale=dev(np.stack([e["entry_scale"] for e in ents])))
        elif efmt == "nvfp4":
            kw = dict(entry_scale=dev(np.stack([e["entry_scale"] for e in ents])))
        if win8 is not None:
            kw["win_scale"] = dev(np.stack([w[1] for w in win8]))
        if roped is not None:
            kw["win_roped"] = True
        out = L.csa_attend(dev(q), e_dev, dev(idx), q_pos0=q_pos0, m=m, win_kv=win, win_pos0=0,
                           n_win=n_win, sink=dev(sk) if sink else None, **kw)
    else:
        out = L.hca_attend(dev(q), e_dev, q_pos0=q_pos0, m=m, win_kv=win, win_pos0=0, n_win=n_win,
                           sink=dev(sk) if sink else None, win_roped=roped is not None)
    torch.cuda.synchronize()
    got = host_bits(out)
    if check_rows is not None:
        rows = np.asarray(check_rows, np.int32)
    if forced_rerun:
        _assert_rerun_forced(forced_rerun, q, kv, ents, sk, rows, heads=sink_heads)
    for b in range(B):
        wkw = dict(win=kv[b] if n_win else None)
        if win8 is not None:
            wkw = dict(win_post=orc.load_window_fp8(*win8[b]))
        if roped is not None:
            wkw = dict(win_post=orc.bf16_to_f64(roped[b]))
        ref = orc.attend_rows(q[b], q_pos0, ents[b]["entries_f64"], m, rows, mode,
                              idx=None if idx is None else idx[b][rows], win_pos0=0, n_win=n_win, sink=sk,
                              **wkw)
        assert_close(got[b][rows], ref, "batch %d" % b)
    return got


def _assert_rerun_forced(kind, q, kv, ents, sk, rows, heads=None):
    """Bounds from the inputs alone.  Dim 0 is never rotated and the rotation
    keeps the norm of the rest, so every logit lambda = <q~, key> / sqrt(128)
    lies within (q_0 key_0 +- |q_1..| |key_1..|) / sqrt(128).  overflow:
    every key's weight against the sink logit is above 2^100, so a row sum
    is too.  underflow (no sink, reference 0): every logit is below
    -80, so the row sum (at most 2^12 keys) is below 2^-100."""
    keys = [np.concatenate([e["entries_f64"], bf16_f64(kv[b])]) for b, e in enumerate(ents)]
    for b, kb in enumerate(keys):
        qb = bf16_f64(q[b][rows])                       # [r, H, 128]
        qn = np.linalg.norm(qb[..., 1:], axis=-1)       # [r, H]
        kn = np.linalg.norm(kb[:, 1:], axis=-1)         # [keys]
        if kind == "overflow":
            lo = (-np.abs(qb[..., 0])[..., None] * np.abs(kb[:, 0]) - qn[..., None] * kn) / np.sqrt(128)
            margin = lo.min(axis=-1) - sk[None, :]      # log weight of the weakest key
            sel = margin if heads is None else margin[:, heads]
            assert sel.min() > 100 * np.log(2), sel.min()
        else:
            assert sk is None
            hi = (qb[..., 0][..., None] * kb[None, None, :, 0] + qn[..., None] * kn) / np.sqrt(128)
            assert hi.max() < -80, hi.max()


@pytest.mark.parametrize("case", [
    dict(B=2, n=77, H=64, q_pos0=50, m=4, mode="csa", k=37),
    dict(B=1, n=64, H=8, q_pos0=300, m=4, mode="csa", k=64, q_scale=24.0),     # sharp logits
    dict(B=1, n=33, H=40, q_pos0=200, m=4, mode="csa", k=70, n_win=0),
    dict(B=1, n=45, H=16, q_pos0=10, m=4, mode="csa", k=8, n_win=5, sink=False),
    dict(B=2, n=50, H=64, q_pos0=400, m=4, mode="csa", k=96, efmt="fp8", kv_scale=1.0),
    dict(B=1, n=300, H=16, q_pos0=0, m=8, mode="hca"),
    dict(B=1, n=129, H=64, q_pos0=2000, m=128, mode="hca", q_scale=24.0),
    dict(B=2, n=40, H=24, q_pos0=700, m=16, mode="hca", n_win=0, sink=False),
    # sink 60 below the scores: weights up to ~2^94 against the sink
    # reference (the bf16 ring kernel stays in range; the FP8 kernel's kSlack
    # restart is what this exercises in the cases further down)
    dict(B=1, n=20, H=32, q_pos0=300, m=4, mode="csa", k=40, sink_shift=-60.0, q_scale=24.0),
    # the ring kernel's max-only rerun: row sums above 2^100 (sink 80 below
    # scores near 0) -- CSA over raw and pre-rotated windows, HCA
    dict(B=2, n=45, H=64, q_pos0=300, m=4, mode="csa", k=40, sink_shift=-80.0, forced_rerun="overflow"),
    dict(B=1, n=45, H=64, q_pos0=300, m=4, mode="csa", k=40, sink_shift=-80.0, wfmt="roped",
         forced_rerun="overflow"),
    dict(B=1, n=60, H=40, q_pos0=900, m=8, mode="hca", sink_shift=-80.0, forced_rerun="overflow"),
    # ... and row sums below 2^-100: no sink, every logit below -80 (keys
    # share +1 on dim 0, queries -1500 there)
    dict(B=1, n=40, H=64, q_pos0=300, m=4, mode="csa", k=40, sink=False, kv_offset=1.0, q_offset=-1500.0,
         forced_rerun="underflow"),
    dict(B=1, n=40, H=32, q_pos0=300, m=4, mode="csa", k=40, sink=False, kv_offset=1.0, q_offset=-1500.0,
         wfmt="roped", forced_rerun="underflow"),
    dict(B=1, n=50, H=64, q_pos0=900, m=8, mode="hca", sink=False, kv_offset=1.0, q_offset=-1500.0,
         forced_rerun="underflow"),
    # only some heads out of range: those rerun, the others keep their pass
    dict(B=1, n=30, H=64, q_pos0=300, m=4, mode="csa", k=40, sink_shift=-80.0,
         sink_heads=np.arange(64) % 3 == 0, forced_rerun="overflow"),
    # sharp logits (q x 128: logit std ~ 1) on the ring kernels
    dict(B=2, n=77, H=64, q_pos0=50, m=4, mode="csa", k=37, q_scale=128.0),
    dict(B=1, n=77, H=64, q_pos0=500, m=4, mode="csa", k=64, q_scale=128.0, wfmt="roped"),
    dict(B=1, n=200, H=64, q_pos0=1000, m=8, mode="hca", q_scale=128.0),
    dict(B=1, n=100, H=16, q_pos0=1000, m=8, mode="hca", q_scale=128.0, wfmt="roped"),
    # FP8 entries with few query rows: each token's 20 chunks are split over
    # 3 work-groups and merged
    dict(B=3, n=2, H=64, q_pos0=2200, m=4, mode="csa", k=512, efmt="fp8", kv_scale=1.0),
    dict(B=2, n=1, H=40, q_pos0=2200, m=4, mode="csa", k=512, efmt="fp8", kv_scale=1.0, sink=False,
         q_scale=24.0),
    dict(B=1, n=3, H=16, q_pos0=2200, m=4, mode="csa", k=500, efmt="fp8", kv_scale=1.0, sink_shift=-60.0,
         q_scale=24.0),
    dict(B=2, n=1, H=64, q_pos0=60, m=4, mode="csa", k=512, efmt="fp8", kv_scale=1.0),  # parts without keys
    # NVFP4 entries (the V4.1 cache variant): many rows, then the split decode
    dict(B=2, n=50, H=64, q_pos0=400, m=4, mode="csa", k=96, efmt="nvfp4", kv_scale=1.0),
    dict(B=3, n=2, H=64, q_pos0=2200, m=4, mode="csa", k=512, efmt="nvfp4", kv_scale=1.0),
    dict(B=1, n=3, H=16, q_pos0=2200, m=4, mode="csa", k=500, efmt="nvfp4", kv_scale=1.0, sink_shift=-60.0,
         q_scale=24.0),
    # the FP8 window cache (V4.1): with NVFP4 and FP8 entries, many rows and the split decode
    dict(B=2, n=50, H=64, q_pos0=400, m=4, mode="csa", k=96, efmt="nvfp4", kv_scale=1.0, wfmt="fp8"),
    dict(B=3, n=2, H=64, q_pos0=2200, m=4, mode="csa", k=512, efmt="nvfp4", kv_scale=1.0, wfmt="fp8"),
    dict(B=2, n=1, H=40, q_pos0=2200, m=4, mode="csa", k=512, efmt="fp8", kv_scale=1.0, wfmt="fp8"),
    # windows rotated once by csa_rope_rows: CSA and HCA ring kernels, the FP8 split decode
    dict(B=2, n=77, H=64, q_pos0=50, m=4, mode="csa", k=37, wfmt="roped"),
    dict(B=1, n=300, H=16, q_pos0=0, m=8, mode="hca", wfmt="roped"),
    dict(B=3, n=2, H=64, q_pos0=2200, m=4, mode="csa", k=512, efmt="fp8", kv_scale=1.0, wfmt="roped"),
])
def test_attend_matches_oracle(orc, case):
    print("attend case %s" % case, flush=True)
    _attend_case(orc, 11, **case)


def test_hca_two_token_work_groups(orc):
    """HCA with at least 4096 query rows, more than 32 heads and at least
    512 entries visible to every row runs two tokens per work-group: one key
    ring for both, each token with its own window chunks, each wave masking
    what its token does not see.  An odd row count leaves the last
    work-group a single token.  The first and last rows, the rows around
    entry-block boundaries and a random sample are checked against the
    oracle."""
    n, m = 2049, 8
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(n - 40, n), np.arange(m - 3, 4 * m + 3),
                                     rng.choice(n, 60, replace=False)]))
    print("hca two-token work-groups", flush=True)
    _attend_case(orc, 12, B=2, n=n, H=40, q_pos0=4200, m=m, mode="hca", check_rows=rows)
    _attend_case(orc, 13, B=1, n=n, H=40, q_pos0=4200, m=m, mode="hca", check_rows=rows, wfmt="roped")


@pytest.mark.parametrize("B,T,pos0", [(2, 300, 0), (1, 257, 1048000)])
def test_rope_rows_matches_oracle(orc, B, T, pos0):
    """csa_rope_rows: dims 0..63 copied, each pair of dims 64..127 rotated at
    its row's position in fp64 and rounded to fp32 then bf16, bit for bit."""
    rng = np.random.default_rng(T)
    kv = _bf16(rng, (B, T, 128), 0.7)
    got = host_bits(L.csa_rope_rows(dev(kv), pos0=pos0))
    for b in range(B):
        assert np.array_equal(got[b], orc.rope_rows_bf16(kv[b], pos0))


def test_attend_deterministic(orc):
    """Run to run bit-identity of one call (batch invariance: test_gpu_invariance.py)."""
    a = _attend_case(orc, 5, B=2, n=40, H=32, q_pos0=100, m=4, mode="csa", k=20)
    b = _attend_case(orc, 5, B=2, n=40, H=32, q_pos0=100, m=4, mode="csa", k=20)
    assert np.array_equal(a, b)


# ------------------------------------------------- config 1, end to end --------

def test_config1_layer_end_to_end(orc):
    """CSA layer, batch 1, 1024 tokens, 8 heads, bf16 indexer (4 heads), k=64:
    compress -> index_topk -> attend on the GPU against the oracle chain."""
    c = synth.config(1)
    print("config 1 end-to-end", flush=True)
    kv, ik, q, qI, w, beta, sink = c["kv"], c["ik"], c["q"], c["q_I"], c["w_I"], c["beta"], c["sink"]
    comp = L.csa_compress(dev(kv), dev(beta), 4, 1, ik=dev(ik), kidx_fmt="bf16")
    idx = L.csa_index_topk(dev(qI), dev(w), comp["kidx"], 64, 4, fmt="bf16")
    out = L.csa_attend(dev(q), comp["entries"], idx, m=4, win_kv=dev(kv), sink=dev(sink))
    torch.cuda.synchronize()
    ref = oracle_compress_store(orc, kv[0], beta, 4, 1, ik=ik[0], kidx_fmt="bf16")
    assert np.array_equal(host_bits(comp["entries"])[0], ref["entries"])
    assert np.array_equal(host_bits(comp["kidx"])[0], ref["kidx"])
    n, N = 1024, 256
    rows = np.arange(n, dtype=np.int32)
    qdec = oracle_q_dec(orc, qI[0], "bf16")
    ref_idx = orc.index_topk_rows(qdec, w[0], ref["kidx_dec"], 4, 0, rows, 64)
    nv = np.minimum(N, (rows + 1) // 4)
    scores = np.zeros((n, N), np.float32)
    for r in range(n):
        scores[r, :nv[r]] = orc.index_scores(qdec[r], w[0, r], ref["kidx_dec"][:nv[r]])
    got_idx = host(idx)[0]
    ndiff = topk_tie_ok(got_idx, ref_idx, scores, nv, 64)
    print("config 1: %d of %d rows differ within the tie band" % (ndiff, n))
    ref_out = orc.attend_rows(q[0], 0, ref["entries_f64"], 4, rows, "csa", idx=ref_idx, win=kv[0],
                              sink=sink)
    mx, mr = assert_close(host_bits(out)[0], ref_out, "config 1")
    print("config 1: max-abs %.3g mean-rel %.3g" % (mx, mr))


# ---------------------------------------------------------- degenerate rows --

@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_attention_rows_without_keys(orc, fmt):
    """Rows whose key set is empty give a zero output, as the oracle's
    softmax over nothing does: HCA rows before the first complete entry with
    no window and no sink, and CSA rows whose top-k slots all hold -1 (bf16
    entries: the ring kernel; FP8 entries with k = 512: the per-token split).
    A row whose only term is the sink is zero too (the sink has no value)."""
    rng = np.random.default_rng(91)
    B, n, H, m = 2, 12, 40, 16
    q = _bf16(rng, (B, n, H, 128), 1 / np.sqrt(128))
    ent = _bf16(rng, (B, 4, 128), 1 / np.sqrt(128))
    win = _bf16(rng, (B, n, 128), 1 / np.sqrt(128))
    sink = rng.standard_normal(H).astype(np.float32)
    # HCA: t = 0 .. 11 < m - 1, so no entry is visible; no window
    for sk in (None, sink):
        out = L.hca_attend(dev(q), dev(ent), q_pos0=0, m=m, win_kv=dev(win), n_win=0,
                           sink=None if sk is None else dev(sk))
        torch.cuda.synchronize()
        got = bf16_f64(host_bits(out))
        assert not np.any(got), "HCA rows without keys (sink %s)" % (sk is not None)
        ref = orc.attend_rows(q[0], 0, orc.bf16_to_f64(ent[0]), m, np.arange(n, dtype=np.int32), "hca",
                              win=win[0], n_win=0, sink=sk)
        assert not np.any(ref), "the oracle's empty rows"
    # CSA: every idx slot -1, no window
    k = 64 if fmt == "bf16" else 512
    N = 600
    idx = np.full((B, n, k), -1, np.int32)
    if fmt == "bf16":
        e = _bf16(rng, (B, N, 128), 1 / np.sqrt(128))
        out = L.csa_attend(dev(q), dev(e), dev(idx), q_pos0=4 * N, m=4, win_kv=dev(win), n_win=0, sink=None)
    else:
        rows = oracle_compress_store(orc, _bf16(rng, (4 * N, 128), 1 / np.sqrt(128)),
                                     rng.standard_normal(8).astype(np.float32), 4, 1, entry_fmt="fp8")
        out = L.csa_attend(dev(q), dev(np.stack([rows["entries"]] * B)), dev(idx), q_pos0=4 * N, m=4,
                           win_kv=dev(win), n_win=0, sink=None,
                           entries_rope=dev(np.stack([rows["entries_rope"]] * B)),
                           entry_scale=dev(np.stack([rows["entry_scale"]] * B)))
    torch.cuda.synchronize()
    assert not np.any(bf16_f64(host_bits(out))), "CSA rows with no selected entry (%s)" % fmt
