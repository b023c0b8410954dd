"""Materialised fp64 NumPy version of the whole layer, for tiny inputs only.

TEST INFRASTRUCTURE ONLY.  It checks the C oracle (``csa_oracle.c``) by a
different construction: pooling as a dense weight matrix, RoPE as complex
multiplication, the indexer as one einsum, top-k by ``np.lexsort``, and
attention as a masked logit matrix with the sink as an extra column.
It follows the same readings of the pages as the C oracle (overlapped
pooling of the previous and current block for CSA [V4-zh 1.1], entries at
their last token, DSA-form indexer, one softmax over sink + entries +
window [V4-wiki, Proposed method item 1]).
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rope_complex(x, pos, rope_dims=64, base=10000.0, sign=1.0):
    """Rotate the last rope_dims dims of x [..., D] by angle pos*theta_f via
    complex multiplication; pos broadcasts against x[..., 0]."""
    x = np.array(x, np.float64, copy=True)
    if rope_dims == 0:
        return x
    D = x.shape[-1]
    f = np.arange(rope_dims // 2, dtype=np.float64)
    theta = base ** (-2.0 * f / rope_dims)
    pos = np.asarray(pos, np.float64)[..., None]
    z = x[..., D - rope_dims::2] + 1j * x[..., D - rope_dims + 1::2]
    z = z * np.exp(1j * sign * pos * theta)
    x[..., D - rope_dims::2] = z.real
    x[..., D - rope_dims + 1::2] = z.imag
    return x


def pooling_matrix(T, m, overlap, beta, z=None):
    """Dense [N, T] matrix of pooling weights (fp64 softmax per entry)."""
    N = T // m
    W = np.zeros((N, T))
    L = 2 * m if overlap else m
    for i in range(N):
        toks, logits = [], []
        for r in range(L):
            if overlap:
                j, role = ((i - 1) * m + r, 1) if r < m else (i * m + r - m, 0)
            else:
                j, role = i * m + r, 0
            if j < 0:
                continue
            toks.append(j)
            logits.append(beta[r] + (0.0 if z is None else z[j, role]))
        lg = np.array(logits)
        e = np.exp(lg - lg.max())
        W[i, toks] += e / e.sum()
    return W


def compress(kv_bits, beta, m, overlap, ik_bits=None, z=None, rope_dims=64, base=10000.0):
    X = bf16_bits_to_f64(kv_bits)
    T = X.shape[0]
    W = pooling_matrix(T, m, overlap, np.asarray(beta, np.float64), z)
    C = W @ X
    p = (np.arange(C.shape[0]) + 1) * m - 1
    C = rope_complex(C, p, rope_dims, base)
    E = None if ik_bits is None else W @ bf16_bits_to_f64(ik_bits)
    return C, E


def index_scores(q, w, keys, relu=True):
    """q [n, H_I, d], w [n, H_I], keys [N, d] -> [n, N] fp64."""
    dots = np.einsum("nhd,sd->nhs", q, keys)
    if relu:
        dots = np.maximum(dots, 0.0)
    return np.einsum("nh,nhs->ns", w, dots)


def topk_rows(scores, n_vis, k):
    """scores [n, N]; row r considers entries [0, n_vis[r]).  Returns [n, k]."""
    out = np.full((scores.shape[0], k), -1, np.int32)
    for r in range(scores.shape[0]):
        nv = int(n_vis[r])
        s = scores[r, :nv]
        order = np.lexsort((np.arange(nv), -s))[:k]
        sel = np.sort(order)
        out[r, :sel.size] = sel
    return out


def attend(q_bits, q_pos0, entries, m, mode, idx=None, win_bits=None, win_pos0=0, n_win=128,
           sink=None, rope_dims=64, base=10000.0):
    """Materialised attention: q [n, H, D] bf16 bits; entries [N, D] fp64
    post-RoPE.  Key set per row = chosen entries + window; logits matrix with
    -inf mask; the sink is an extra logit column with a zero value."""
    Q = bf16_bits_to_f64(q_bits)
    n, H, D = Q.shape
    t = q_pos0 + np.arange(n)
    Qr = rope_complex(Q, t[:, None], rope_dims, base)
    N = entries.shape[0]
    if win_bits is not None and n_win > 0:
        Wr = bf16_bits_to_f64(win_bits)
        jpos = win_pos0 + np.arange(Wr.shape[0])
        Wr = rope_complex(Wr, jpos, rope_dims, base)
    else:
        Wr = np.zeros((0, D))
        jpos = np.zeros((0,), np.int64)
    Kall = np.concatenate([entries, Wr], axis=0)
    mask = np.zeros((n, Kall.shape[0]), bool)
    p_ent = (np.arange(N) + 1) * m - 1
    for r in range(n):
        if mode == "csa":
            sel = idx[r][idx[r] >= 0]
            mask[r, sel] = True
        else:
            mask[r, :N] = p_ent <= t[r]
        if Wr.shape[0]:
            mask[r, N:] = (jpos <= t[r]) & (jpos >= t[r] - n_win + 1) & (jpos >= 0)
    logits = np.einsum("nhd,kd->nhk", Qr, Kall) / np.sqrt(D)
    logits = np.where(mask[:, None, :], logits, -np.inf)
    if sink is not None:
        sk = np.broadcast_to(np.asarray(sink, np.float64)[None, :, None], (n, H, 1))
        logits = np.concatenate([logits, sk], axis=2)
        V = np.concatenate([Kall, np.zeros((1, D))], axis=0)
    else:
        V = Kall
    mx = logits.max(axis=2, keepdims=True)
    P = np.exp(logits - mx)
    P = P / P.sum(axis=2, keepdims=True)
    O = np.einsum("nhk,kd->nhd", P, V)
    return rope_complex(O, t[:, None], rope_dims, base, sign=-1.0)
