"""MI355X-native hybrid compressed attention forward (CSA + HCA).

Python binding of the C ABI in include/csa.h.  Every function here only
marshals arguments: torch tensors supply device memory and the current HIP
stream; every step of the computation runs in the HIP kernels of
``libcsa_mi355x.so``.  Output tensors are allocated with torch when the
caller does not pass them.

Names follow the C ABI: csa_compress, csa_cache_append, csa_index_topk,
csa_attend, csa_index_attend (the two pipelined over token chunks), hca_attend, and the projections around the path
(csa_project_in, csa_project_qidx, csa_project_out).
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import (FMT_BF16, FMT_BF16_ROPED, FMT_FP8, FMT_FP8_ROPE_BF16, FMT_MXFP4, FMT_NVFP4, CsaError, check,
                   lib)

__all__ = ["csa_compress", "csa_cache_append", "csa_index_topk", "csa_index_topk_noalloc", "csa_attend",
           "csa_index_attend", "hca_attend",
           "csa_project_in", "csa_project_qidx", "csa_project_out", "csa_rope_rows", "version",
           "CsaError",
           "FMT_BF16", "FMT_MXFP4", "FMT_FP8_ROPE_BF16", "FMT_NVFP4", "FMT_FP8"]

_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _fmt(name):
    return {"bf16": FMT_BF16, "mxfp4": FMT_MXFP4, "fp8": FMT_FP8_ROPE_BF16, "nvfp4": FMT_NVFP4}[name]


def version():
    return lib().csa_version()


def csa_compress(kv, beta, m, overlap, pos0=0, ik=None, z=None, prev_kv=None, prev_ik=None,
                 prev_z=None, rope_dims=64, rope_base=10000.0, entry_fmt="bf16", kidx_fmt="mxfp4",
                 out=None, stream=None):
    """kv [B, T, 128] bf16 -> dict(entries, entries_rope, entry_scale, kidx, kidx_scale).
    entry_fmt "bf16", "fp8" (e4m3 + bf16 RoPE dims + scale) or "nvfp4"
    (records [B, N, 72] u8 + scale).
    ``out`` may hold preallocated output tensors under the same keys (e.g.
    views into a larger cache)."""
    B, T, D = kv.shape
    n_new = T // m
    dev = kv.device
    out = dict(out or {})
    ef, kf = _fmt(entry_fmt), _fmt(kidx_fmt)
    if "entries" not in out:
        if ef == FMT_BF16:
            out["entries"] = torch.empty((B, n_new, D), dtype=torch.bfloat16, device=dev)
        else:
            out["entries"] = torch.empty((B, n_new, 72 if ef == FMT_NVFP4 else 64), dtype=torch.uint8, device=dev)
    if ef == FMT_FP8_ROPE_BF16:
        out.setdefault("entries_rope", torch.empty((B, n_new, 64), dtype=torch.bfloat16, device=dev))
    if ef in (FMT_FP8_ROPE_BF16, FMT_NVFP4):
        out.setdefault("entry_scale", torch.empty((B, n_new), dtype=torch.float32, device=dev))
    if ik is not None:
        if kf == FMT_BF16:
            out.setdefault("kidx", torch.empty((B, n_new, 64), dtype=torch.bfloat16, device=dev))
        else:
            out.setdefault("kidx", torch.empty((B, n_new, 32), dtype=torch.uint8, device=dev))
            out.setdefault("kidx_scale", torch.empty((B, n_new, 2), dtype=torch.uint8, device=dev))
    check(lib().csa_compress(
        _ptr(kv), _ptr(ik), _ptr(z), _ptr(beta), _ptr(prev_kv), _ptr(prev_ik), _ptr(prev_z),
        B, T, int(pos0), D, 64 if ik is not None else 0, m, int(overlap), rope_dims,
        float(rope_base), _ptr(out["entries"]), _ptr(out.get("entries_rope")),
        _ptr(out.get("entry_scale")), ef, _ptr(out.get("kidx")), _ptr(out.get("kidx_scale")), kf,
        _stream(stream)))
    return out


def csa_cache_append(kv_new, beta, m, overlap, t, kv_ring, caches, ik_new=None, ik_ring=None,
                     z_new=None, z_ring=None, rope_dims=64, rope_base=10000.0, entry_fmt="bf16",
                     kidx_fmt="mxfp4", win8_ring=None, win8_scale=None, stream=None):
    """Decode write path: kv_new [B, 128] (ik_new [B, 64], z_new [B, 2]) of
    position t into the rings kv_ring [B, 2W, 128] (ik_ring [B, W, 64],
    z_ring [B, W, 2]); the block it completes, if any, into ``caches``
    (entries [B, N_cap, ...], entries_rope, entry_scale, kidx, kidx_scale).
    win8_ring [B, 2W, 128] u8 + win8_scale [B, 2W] f32: optional FP8 window
    cache (rows rotated at their positions), slots as kv_ring."""
    B = kv_new.shape[0]
    W = kv_ring.shape[1] // 2
    ents = caches.get("entries")
    N_cap = 0 if ents is None else ents.shape[1]
    check(lib().csa_cache_append(
        _ptr(kv_new), _ptr(ik_new), _ptr(z_new), B, int(t), _ptr(kv_ring), _ptr(ik_ring), _ptr(z_ring),
        _ptr(win8_ring), _ptr(win8_scale), W,
        _ptr(beta), m, int(overlap), rope_dims, float(rope_base), _ptr(ents), _ptr(caches.get("entries_rope")),
        _ptr(caches.get("entry_scale")), _fmt(entry_fmt), _ptr(caches.get("kidx")), _ptr(caches.get("kidx_scale")),
        _fmt(kidx_fmt), N_cap, _stream(stream)))


def csa_index_topk(qidx, widx, kidx, k, m, q_pos0=0, fmt="mxfp4", qidx_scale=None,
                   kidx_scale=None, N=None, idx_out=None, ws=None, fallback_count=None, stream=None):
    """qidx [B, n, H_I, 64] bf16 (or [B, n, H_I, 32] MXFP4 codes with
    qidx_scale), widx [B, n, H_I] fp32, kidx [B, N, 64|32] -> idx [B, n, k]
    int32, each row's indices ascending.  fallback_count: an optional int32
    cuda tensor of one element, to which the kernels add the number of
    work-groups that took the exact streaming path (the caller clears it)."""
    B, n, H_I = qidx.shape[:3]
    if N is None:
        N = kidx.shape[1]
    f = _fmt(fmt)
    if idx_out is None:
        idx_out = torch.empty((B, n, k), dtype=torch.int32, device=qidx.device)
    need = lib().csa_index_topk_workspace_bytes(B, n, int(q_pos0), N, m, k)
    if ws is None and need > 0:
        ws = torch.empty((need,), dtype=torch.uint8, device=qidx.device)
    check(lib().csa_index_topk(
        _ptr(qidx), _ptr(qidx_scale), _ptr(widx), _ptr(kidx), _ptr(kidx_scale), f, B, n,
        int(q_pos0), H_I, 64, N, m, k, _ptr(idx_out), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _ptr(fallback_count), _stream(stream)))
    return idx_out


def csa_index_topk_noalloc(qidx, widx, kidx, k, m, idx_out, q_pos0=0, fmt="mxfp4", qidx_scale=None,
                           kidx_scale=None, N=None, fallback_count=None, stream=None):
    """csa_index_topk without a workspace (csa_index_topk_noalloc): the
    split path uses the library's static device scratch (at most 256 split
    rows); the caller passes idx_out and the call allocates nothing."""
    B, n, H_I = qidx.shape[:3]
    if N is None:
        N = kidx.shape[1]
    check(lib().csa_index_topk_noalloc(
        _ptr(qidx), _ptr(qidx_scale), _ptr(widx), _ptr(kidx), _ptr(kidx_scale), _fmt(fmt), B, n,
        int(q_pos0), H_I, 64, N, m, k, _ptr(idx_out), _ptr(fallback_count), _stream(stream)))
    return idx_out


def csa_attend(q, entries, idx, q_pos0=0, m=4, win_kv=None, win_pos0=0, n_win=128, sink=None,
               entries_rope=None, entry_scale=None, rope_dims=64, rope_base=10000.0, N=None,
               out=None, ws=None, win_scale=None, win_roped=False, stream=None):
    """q [B, n, H, 128] bf16; entries [B, N, 128] bf16 (or e4m3 [B, N, 64] with
    entries_rope/entry_scale, or NVFP4 records [B, N, 72] u8 with entry_scale
    only); idx [B, n, k] int32; win_kv [B, W, 128] bf16 raw rows, or with
    win_scale an FP8 window cache (e4m3 [B, W, 128] of rotated rows), or
    with win_roped rows rotated by csa_rope_rows.
    ``ws``: workspace of csa_attend_workspace_bytes() bytes (allocated here
    when needed and not given)."""
    B, n, H, D = q.shape
    if N is None:
        N = entries.shape[1]
    if entries_rope is not None:
        ef = FMT_FP8_ROPE_BF16
    elif entry_scale is not None:
        ef = FMT_NVFP4  # NVFP4 records [B, N, 72] u8 + entry_scale
    else:
        ef = FMT_BF16
    want = {FMT_BF16: D, FMT_FP8_ROPE_BF16: 64, FMT_NVFP4: 72}[ef]
    if entries.shape[-1] != want:
        raise ValueError("csa_attend: entries of the %s format have %d values per row, got %d"
                         % ({FMT_BF16: "bf16", FMT_FP8_ROPE_BF16: "fp8", FMT_NVFP4: "nvfp4"}[ef], want,
                            entries.shape[-1]))
    if out is None:
        out = torch.empty_like(q, dtype=torch.bfloat16)
    win_len = 0 if win_kv is None else win_kv.shape[1]
    nw = int(n_win) if win_kv is not None else 0
    need = lib().csa_attend_workspace_bytes(B, n, idx.shape[2], nw, ef)
    if ws is None and need > 0:
        ws = torch.empty((need,), dtype=torch.uint8, device=q.device)
    check(lib().csa_attend(
        _ptr(q), B, n, int(q_pos0), H, D, _ptr(entries), _ptr(entries_rope), _ptr(entry_scale), ef,
        N, m, _ptr(idx), idx.shape[2], _ptr(win_kv), int(win_pos0), win_len, nw,
        FMT_FP8 if win_scale is not None else (FMT_BF16_ROPED if win_roped else FMT_BF16), _ptr(win_scale),
        _ptr(sink), rope_dims,
        float(rope_base), _ptr(out), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)))
    return out


_pipes = {}


def _pipe(device):
    """The aux stream and three events csa_index_attend runs its chunks
    with, one set per device, created on first use (each event recorded
    once so that its HIP handle exists)."""
    key = torch.device(device).index
    if key not in _pipes:
        aux = torch.cuda.Stream(device=device)
        evs = [torch.cuda.Event() for _ in range(3)]
        for e in evs:
            e.record(aux)
        _pipes[key] = (aux, evs, (ctypes.c_void_p * 3)(*[e.cuda_event for e in evs]))
    return _pipes[key]


def csa_index_attend(qidx, widx, kidx, k, m, q, entries, q_pos0=0, fmt="mxfp4", qidx_scale=None,
                     kidx_scale=None, N=None, idx_out=None, fallback_count=None, win_kv=None, win_pos0=0,
                     n_win=128, sink=None, entries_rope=None, entry_scale=None, rope_dims=64, rope_base=10000.0,
                     out=None, win_scale=None, win_roped=False, n_chunks=16, aux_stream=None, stream=None):
    """csa_index_topk then csa_attend (arguments as there), pipelined over
    n_chunks chunks of query tokens: the indexer of a chunk runs on an aux
    stream beside the attention of the one before, on ``stream``.  Returns
    (idx_out, out); both are the bytes the two separate calls write."""
    B, n, H, D = q.shape
    H_I = qidx.shape[2]
    if N is None:
        N = entries.shape[1]
    if entries_rope is not None:
        ef = FMT_FP8_ROPE_BF16
    elif entry_scale is not None:
        ef = FMT_NVFP4
    else:
        ef = FMT_BF16
    if idx_out is None:
        idx_out = torch.empty((B, n, k), dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty_like(q, dtype=torch.bfloat16)
    aux, _, evs = _pipe(q.device)
    if aux_stream is not None:
        aux = aux_stream
    win_len = 0 if win_kv is None else win_kv.shape[1]
    nw = int(n_win) if win_kv is not None else 0
    wf = FMT_FP8 if win_scale is not None else (FMT_BF16_ROPED if win_roped else FMT_BF16)
    check(lib().csa_index_attend(
        _ptr(qidx), _ptr(qidx_scale), _ptr(widx), _ptr(kidx), _ptr(kidx_scale), _fmt(fmt), H_I, 64, k,
        _ptr(idx_out), _ptr(fallback_count), _ptr(q), H, D, _ptr(entries), _ptr(entries_rope), _ptr(entry_scale),
        ef, _ptr(win_kv), int(win_pos0), win_len, nw, wf, _ptr(win_scale), _ptr(sink), rope_dims, float(rope_base),
        _ptr(out), B, n, int(q_pos0), N, m, int(n_chunks), _stream(stream), aux.cuda_stream, evs))
    return idx_out, out


def hca_attend(q, entries, q_pos0=0, m=128, win_kv=None, win_pos0=0, n_win=128, sink=None,
               rope_dims=64, rope_base=10000.0, N=None, out=None, win_roped=False, stream=None):
    """q [B, n, H, 128] bf16; entries [B, N, 128] bf16: dense attention over
    every visible entry + window + sink.  win_roped: win_kv rows were rotated
    by csa_rope_rows."""
    B, n, H, D = q.shape
    if N is None:
        N = entries.shape[1]
    if out is None:
        out = torch.empty_like(q, dtype=torch.bfloat16)
    win_len = 0 if win_kv is None else win_kv.shape[1]
    check(lib().hca_attend(
        _ptr(q), B, n, int(q_pos0), H, D, _ptr(entries), N, m, _ptr(win_kv), int(win_pos0), win_len,
        int(n_win) if win_kv is not None else 0, FMT_BF16_ROPED if win_roped else FMT_BF16, _ptr(sink),
        rope_dims, float(rope_base), _ptr(out), _stream(stream)))
    return out


def csa_project_in(x, w_in, widths, w_up=None, n_qidx=0, out=None, stream=None):
    """Input projections (csa_project_in).  x [..., d] bf16; w_in
    [sum(widths), d] bf16 = W_q, W_kv, W_ik, W_lat, W_w, W_z stacked; widths =
    (n_q, n_kv, n_ik, n_lat, n_w, n_z); w_up [n_qidx, n_lat] bf16.  Returns a
    dict of q, kv, ik, lat (bf16 [M, n_*]), w and z (fp32 [M, n_w], [M, n_z])
    and, when n_qidx > 0, qidx (uint8 [M, n_qidx/2]) and qidx_scale (uint8
    [M, n_qidx/32]); M = x.numel() / d.  Widths of 0 give no tensor."""
    d = x.shape[-1]
    M = x.numel() // d
    n_q, n_kv, n_ik, n_lat, n_w, n_z = widths
    dev = x.device
    out = dict(out or {})
    for name, n, dt in (("q", n_q, torch.bfloat16), ("kv", n_kv, torch.bfloat16), ("ik", n_ik, torch.bfloat16),
                        ("lat", n_lat, torch.bfloat16), ("w", n_w, torch.float32), ("z", n_z, torch.float32)):
        if n and name not in out:
            out[name] = torch.empty((M, n), dtype=dt, device=dev)
    if n_qidx:
        out.setdefault("qidx", torch.empty((M, n_qidx // 2), dtype=torch.uint8, device=dev))
        out.setdefault("qidx_scale", torch.empty((M, n_qidx // 32), dtype=torch.uint8, device=dev))
    check(lib().csa_project_in(_ptr(x), M, d, _ptr(w_in), n_q, n_kv, n_ik, n_lat, n_w, n_z, _ptr(w_up), n_qidx,
                               _ptr(out.get("q")), _ptr(out.get("kv")), _ptr(out.get("ik")), _ptr(out.get("lat")),
                               _ptr(out.get("w")), _ptr(out.get("z")), _ptr(out.get("qidx")),
                               _ptr(out.get("qidx_scale")),
                               _stream(stream)))
    return out


def csa_project_qidx(lat, w_up, with_f32=False, stream=None):
    """The indexer-query step (csa_project_qidx): lat [M, r] bf16, w_up
    [n_qidx, r] bf16 -> (codes uint8 [M, n_qidx/2], scales uint8
    [M, n_qidx/32], fp32 values [M, n_qidx] or None)."""
    M, r = lat.shape
    n_qidx = w_up.shape[0]
    codes = torch.empty((M, n_qidx // 2), dtype=torch.uint8, device=lat.device)
    scales = torch.empty((M, n_qidx // 32), dtype=torch.uint8, device=lat.device)
    qf = torch.empty((M, n_qidx), dtype=torch.float32, device=lat.device) if with_f32 else None
    check(lib().csa_project_qidx(_ptr(lat), M, r, _ptr(w_up), n_qidx, _ptr(codes), _ptr(scales), _ptr(qf),
                                 _stream(stream)))
    return codes, scales, qf


def csa_project_out(o, w_o, G, out=None, stream=None):
    """Grouped output projection (csa_project_out): o [..., H, D] bf16,
    w_o [d, (H/G)*D] bf16 -> y [M, d] bf16 (M = o.numel() / (H*D))."""
    H, D = o.shape[-2], o.shape[-1]
    M = o.numel() // (H * D)
    d = w_o.shape[0]
    if out is None:
        out = torch.empty((M, d), dtype=torch.bfloat16, device=o.device)
    check(lib().csa_project_out(_ptr(o), M, H, D, G, _ptr(w_o), d, _ptr(out), _stream(stream)))
    return out


def csa_rope_rows(kv, pos0=0, rope_dims=64, rope_base=10000.0, out=None, stream=None):
    """kv [B, T, 128] bf16 raw rows of positions pos0.. -> the rows rotated
    at their positions (csa_rope_rows), for win_roped windows."""
    B, T, _ = kv.shape
    if out is None:
        out = torch.empty_like(kv)
    check(lib().csa_rope_rows(_ptr(kv), B, T, int(pos0), rope_dims, float(rope_base), _ptr(out), _stream(stream)))
    return out
