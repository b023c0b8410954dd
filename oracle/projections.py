"""CPU oracle for the projections around the attention path (hidden state in,
grouped output projection out).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: imported by
``tests/`` and ``bench.py``'s cpu_baseline leg, never by the library.

What the pages fix: "DeepSeek-V4: Towards Highly Efficient Million-Token
Context Intelligence" wiki summary, Proposed method item 1 (CSA uses a
shared-KV multi-query attention and a grouped output projection; the
Lightning Indexer is cheap through a low-rank factorisation and FP4
arithmetic, "deepseek V4 技术论文" 1.1; hidden sizes 7168 / 4096 in the
model list) and Post-training item 3 (the indexer's QK path in MXFP4).
Everything else is a reading, stated where it is used:

* P1  every projection is a plain linear map without bias, weights in the
      [out, in] layout; products are exact (bf16 x bf16) and summed in
      fp64 here (numpy matmul is the library step), then rounded to fp32
      (RNE) -- the value a kernel accumulating in fp32 aims at -- and, for
      the bf16 outputs (q, kv, ik and the indexer latent), on to bf16 RNE;
      the indexer head weights w_I stay fp32.
* P2  the indexer query is low rank: q_I = lat . W_up^T with lat the bf16
      latent (rank r) and W_up [H_I*64, r]; the fp32 value of q_I is then
      MXFP4-encoded per 32-element block with the O4 rule.
* P4  the compression logits z (the per-token slot-logit offsets the
      compressor adds to its learned bias) are one more linear map of the
      hidden state, kept in fp32 like w_I.
* P3  the grouped output projection splits the H heads into G groups of
      consecutive heads; group j's head outputs (H/G x 128 values) are
      projected by its own [d/G, (H/G)*128] block onto output columns
      [j*d/G, (j+1)*d/G).  Nothing mixes the groups (a block-diagonal map,
      as in a grouped convolution).  bf16 result.

The arithmetic is numpy fp64; the MXFP4 encoder is the pinned one of
``oracle.mxfp4_encode``.
"""
from __future__ import annotations

import numpy as np

from . import bf16_from_f32, bf16_to_f64, mxfp4_encode


def _f64(bits):
    return bf16_to_f64(np.ascontiguousarray(bits, np.uint16))


def linear_f64(x_bits, w_bits):
    """x [M, K] and w [N, K] as bf16 bits -> x . w^T in fp64 (P1)."""
    return _f64(x_bits) @ _f64(w_bits).T


def _bf16(y64):
    # fp64 -> fp32 (RNE) -> bf16 (RNE): the fp64 sum of exact products,
    # rounded as the kernels round their fp32 result
    return bf16_from_f32(y64.astype(np.float32))


def project_in(x, w_q, w_kv, w_ik, w_lat, w_w, w_up, w_z=None):
    """The input projections of one layer (P1, P2, P4).

    x [M, d] bf16 bits; w_q [H*128, d], w_kv [128, d], w_ik [64, d],
    w_lat [r, d], w_w [H_I, d], w_up [H_I*64, r], all bf16 bits.
    Returns dict: q [M, H*128] bf16, kv [M, 128] bf16, ik [M, 64] bf16,
    lat [M, r] bf16, w_I [M, H_I] fp32, q_I codes [M, H_I*32] uint8 and
    q_I scales [M, H_I*2] uint8 (MXFP4), and q_I_f32 [M, H_I*64] (the fp32
    values that were encoded); with w_z [n_z, d], also z [M, n_z] fp32."""
    out = {
        "q": _bf16(linear_f64(x, w_q)),
        "kv": _bf16(linear_f64(x, w_kv)),
        "ik": _bf16(linear_f64(x, w_ik)),
        "lat": _bf16(linear_f64(x, w_lat)),
        "w_I": linear_f64(x, w_w).astype(np.float32),
    }
    if w_z is not None:
        out["z"] = linear_f64(x, w_z).astype(np.float32)
    qf = linear_f64(out["lat"], w_up).astype(np.float32)
    codes, scales = mxfp4_encode(qf)
    out["q_I_f32"] = qf
    out["q_I_codes"] = codes
    out["q_I_scales"] = scales
    return out


def project_out(o, w_o, G):
    """Grouped output projection (P3).  o [M, H*128] bf16 bits (head-major
    rows), w_o [d, (H/G)*128] bf16 bits with group j's block in rows
    [j*d/G, (j+1)*d/G).  Returns y [M, d] bf16 and its fp64 value."""
    o64 = _f64(o)
    w64 = _f64(w_o)
    M, HD = o64.shape
    d, KG = w64.shape
    assert HD == G * KG and d % G == 0
    dg = d // G
    y = np.empty((M, d), np.float64)
    for j in range(G):
        y[:, j * dg:(j + 1) * dg] = o64[:, j * KG:(j + 1) * KG] @ w64[j * dg:(j + 1) * dg].T
    return _bf16(y), y
