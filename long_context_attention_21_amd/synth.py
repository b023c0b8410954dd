"""Seeded synthetic inputs for the hybrid compressed attention forward.

This module holds no arithmetic of the method: it only draws random numbers
in a fixed order (``numpy.random.default_rng(seed)``, float32 standard
normals times a scale), rounds them to bf16 and shapes them.  Both the HIP
path and the CPU oracle consume what it returns, so it is the one piece of
code they share.  Quantised inputs (FP8 / MXFP4 caches) are *not* produced
here: the caller encodes the raw draws with its own encoder.

Workloads (the five configurations of the hot path):
  1  CSA layer, batch 1, 1024 tokens, 8 heads, indexer 4 heads bf16, k = 64
  2  HCA layer, batch 1, 32768 tokens, 64 heads, m' = 128
  3  CSA prefill, batch 1, 131072 tokens, 64 heads, MXFP4 indexer 8 heads, k = 2048
  4  CSA decode, 64 sequences x 262144 cached entries (FP8 + bf16), k = 2048
  5  CSA + HCA layer pair, 8192 new tokens after 1,048,576 prior tokens
"""
from __future__ import annotations

import math

import numpy as np

D_HEAD = 128
ROPE_DIMS = 64
ROPE_BASE = 10000.0
N_WIN = 128
D_IDX = 64

_CHUNK = 1 << 26


def normal(rng, shape, scale=1.0):
    """float32 N(0,1) * scale, drawn in consecutive chunks (same stream as one
    draw) to bound peak host memory."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
        if scale != 1.0:
            out[s:e] *= np.float32(scale)
    return out.reshape(shape)


def to_bf16_bits(x):
    """float32 -> bf16 bit patterns (uint16), round to nearest even, via torch."""
    import torch
    x = np.ascontiguousarray(x, np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, np.uint16)
    for s in range(0, flat.size, _CHUNK):
        e = min(flat.size, s + _CHUNK)
        t = torch.from_numpy(flat[s:e]).to(torch.bfloat16)
        out[s:e] = t.view(torch.int16).numpy().view(np.uint16)
    return out.reshape(x.shape)


def normal_bf16(rng, shape, scale=1.0):
    """Draw in chunks and round each chunk to bf16 at once (no full fp32 copy)."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[s:e] = to_bf16_bits(x)
    return out.reshape(shape)


def csa_prefill(n, H, H_I, rank, k, seed, B=1, m=4, indexer="mxfp4", q_scale=1.0,
                with_z=False, q_pos0=0):
    """CSA layer inputs (configurations 1 and 3, and scaled-down variants).

    Draw order: q, kv, ik, beta, latent, W_up, w_I, sink (, z).  q_I is the
    caller-side low-rank up-projection latent @ W_up in fp32, rounded to bf16.
    """
    rng = np.random.default_rng(seed)
    D, d = D_HEAD, D_IDX
    q = normal_bf16(rng, (B, n, H, D), q_scale / math.sqrt(D))
    kv = normal_bf16(rng, (B, n, D), 1 / math.sqrt(D))
    ik = normal_bf16(rng, (B, n, d), 1 / math.sqrt(d))
    beta = normal(rng, (2 * m,))
    lat = normal(rng, (B, n, rank), 1 / math.sqrt(rank))
    w_up = normal(rng, (rank, H_I * d), 1 / math.sqrt(rank))
    w_I = normal(rng, (B, n, H_I), 1 / math.sqrt(H_I))
    sink = normal(rng, (H,))
    z = normal(rng, (B, n, 2)) if with_z else None
    q_I = np.empty((B, n, H_I, d), np.uint16)
    step = 1 << 16
    for b in range(B):
        for s in range(0, n, step):
            e = min(n, s + step)
            q_I[b, s:e] = to_bf16_bits((lat[b, s:e] @ w_up).reshape(e - s, H_I, d))
    return dict(kind="csa", B=B, n=n, H=H, D=D, H_I=H_I, d_idx=d, m=m, overlap=1, k=k,
                n_win=N_WIN, q_pos0=q_pos0, indexer=indexer, q=q, kv=kv, ik=ik, beta=beta,
                q_I=q_I, w_I=w_I, sink=sink, z=z)


def hca_prefill(n, H, seed, B=1, m=128, q_scale=1.0, q_pos0=0):
    """HCA layer inputs (configuration 2).  Draw order: q, kv, beta, sink."""
    rng = np.random.default_rng(seed)
    D = D_HEAD
    q = normal_bf16(rng, (B, n, H, D), q_scale / math.sqrt(D))
    kv = normal_bf16(rng, (B, n, D), 1 / math.sqrt(D))
    beta = normal(rng, (m,))
    sink = normal(rng, (H,))
    return dict(kind="hca", B=B, n=n, H=H, D=D, m=m, overlap=0, n_win=N_WIN, q_pos0=q_pos0,
                q=q, kv=kv, beta=beta, sink=sink)


def decode_raw(B, N, H, H_I, k, seed, n_win=N_WIN, q_scale=1.0):
    """CSA decode inputs (configuration 4), raw draws only.

    Per sequence b in order: entries [N, 128] N(0,1) fp32, indexer keys
    [N, 64] N(0,1) fp32, SWA cache [n_win, 128] N(0,1) -> bf16.  Then q
    [B, 1, H, 128] / sqrt(128), q_I [B, 1, H_I, 64] / sqrt(64), w_I
    [B, 1, H_I] / sqrt(H_I), sink [H].  ``seq(b)`` yields sequence b's raw
    draws; it must be called for b = 0, 1, ... in order (one stream).
    The caller quantises entries (FP8 dims 0..63 + bf16 RoPE dims) and keys
    (MXFP4) with its own encoder.  The query sits at t = 4N (all entries
    visible) and the SWA cache holds positions t-n_win+1 .. t.
    """
    rng = np.random.default_rng(seed)
    state = {"next": 0}

    def seq(b):
        assert b == state["next"], "sequences must be drawn in order"
        state["next"] += 1
        ent = normal(rng, (N, D_HEAD))
        ik = normal(rng, (N, D_IDX))
        swa = normal_bf16(rng, (n_win, D_HEAD))
        return ent, ik, swa

    def tail():
        assert state["next"] == B, "draw every sequence first"
        q = normal_bf16(rng, (B, 1, H, D_HEAD), q_scale / math.sqrt(D_HEAD))
        q_I = normal_bf16(rng, (B, 1, H_I, D_IDX), 1 / math.sqrt(D_IDX))
        w_I = normal(rng, (B, 1, H_I), 1 / math.sqrt(H_I))
        sink = normal(rng, (H,))
        return q, q_I, w_I, sink

    t = 4 * N
    return dict(kind="decode", B=B, N=N, H=H, H_I=H_I, d_idx=D_IDX, m=4, k=k, n_win=n_win,
                q_pos0=t, win_pos0=t - n_win + 1, seq=seq, tail=tail)


def pair_chunk(n_new, N_csa_prior, N_hca_prior, H, H_I, rank, k, seed, q_scale=1.0,
               zipf_s=1.1):
    """Chunked-prefill CSA + HCA layer pair (configuration 5).

    The chunk starts at P = 4 * N_csa_prior (= 128 * N_hca_prior).
    CSA draws: entries_prior, kI_prior, Zipf rank permutation, state_kv
    (positions P-128..P-1), state_ik (P-4..P-1), kv_new, ik_new, beta,
    latent, W_up, w_I, q, sink.  HCA draws: entries_prior, state_kv, kv_new,
    beta, q, sink.  The Zipf multiplier (rank/k)^(-s) scales the prior
    indexer-key rows only.
    """
    assert 4 * N_csa_prior == 128 * N_hca_prior
    P = 4 * N_csa_prior
    rng = np.random.default_rng(seed)
    D, d = D_HEAD, D_IDX
    c = {}
    c["entries_prior"] = normal_bf16(rng, (N_csa_prior, D), 1 / math.sqrt(D))
    kI = normal(rng, (N_csa_prior, d), 1 / math.sqrt(d))
    rank_perm = rng.permutation(N_csa_prior) + 1
    mult = (rank_perm.astype(np.float64) / k) ** (-zipf_s)
    c["kI_prior_f32"] = (kI * mult[:, None].astype(np.float32)).astype(np.float32)
    c["state_kv"] = normal_bf16(rng, (N_WIN, D), 1 / math.sqrt(D))
    c["state_ik"] = normal_bf16(rng, (4, d), 1 / math.sqrt(d))
    c["kv_new"] = normal_bf16(rng, (n_new, D), 1 / math.sqrt(D))
    c["ik_new"] = normal_bf16(rng, (n_new, d), 1 / math.sqrt(d))
    c["beta"] = normal(rng, (8,))
    lat = normal(rng, (n_new, rank), 1 / math.sqrt(rank))
    w_up = normal(rng, (rank, H_I * d), 1 / math.sqrt(rank))
    c["w_I"] = normal(rng, (n_new, H_I), 1 / math.sqrt(H_I))
    c["q"] = normal_bf16(rng, (n_new, H, D), q_scale / math.sqrt(D))
    c["sink"] = normal(rng, (H,))
    c["q_I"] = to_bf16_bits((lat @ w_up).reshape(n_new, H_I, d))
    h = {}
    h["entries_prior"] = normal_bf16(rng, (N_hca_prior, D), 1 / math.sqrt(D))
    h["state_kv"] = normal_bf16(rng, (N_WIN, D), 1 / math.sqrt(D))
    h["kv_new"] = normal_bf16(rng, (n_new, D), 1 / math.sqrt(D))
    h["beta"] = normal(rng, (128,))
    h["q"] = normal_bf16(rng, (n_new, H, D), q_scale / math.sqrt(D))
    h["sink"] = normal(rng, (H,))
    return dict(kind="pair", n=n_new, P=P, H=H, H_I=H_I, d_idx=d, k=k, n_win=N_WIN,
                N_csa_prior=N_csa_prior, N_hca_prior=N_hca_prior, csa=c, hca=h)


def config(i, q_scale=1.0):
    """The five workloads at full size."""
    if i == 1:
        return csa_prefill(1024, 8, 4, 32, 64, seed=0, indexer="bf16", q_scale=q_scale)
    if i == 2:
        return hca_prefill(32768, 64, seed=1, q_scale=q_scale)
    if i == 3:
        return csa_prefill(131072, 64, 8, 32, 2048, seed=2, indexer="mxfp4", q_scale=q_scale)
    if i == 4:
        return decode_raw(64, 262144, 64, 8, 2048, seed=3, q_scale=q_scale)
    if i == 5:
        return pair_chunk(8192, 262144, 8192, 64, 8, 32, 2048, seed=4, q_scale=q_scale)
    raise ValueError(i)
