"""CPU oracle for the hybrid compressed attention forward (CSA + HCA).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``.  The library in
``long_context_attention_21_amd`` never imports it and shares no code with it.

This module is a thin ctypes wrapper around ``csa_oracle.c`` (the arithmetic
lives there, each function citing the passage of the pages it follows).  All
arrays are host numpy arrays; bf16 tensors are ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libcsa_oracle.so")
_SRC = os.path.join(_HERE, "csa_oracle.c")

GCC_FLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11",
             "-Wall", "-Wextra"]


def build(force: bool = False) -> str:
    """Compile csa_oracle.c into libcsa_oracle.so (plain gcc, no fast-math)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = C.CDLL(_SO)
        P = C.c_void_p
        i32, i64, dbl = C.c_int, C.c_int64, C.c_double
        sig = {
            "orc_bf16_from_f32_n": (None, [P, i64, P]),
            "orc_bf16_to_f64_n": (None, [P, i64, P]),
            "orc_e4m3_from_f32_n": (None, [P, i64, P]),
            "orc_e4m3_to_f32_n": (None, [P, i64, P]),
            "orc_store_entries_fp8_n": (None, [P, i64, i32, i32, P, P, P]),
            "orc_load_entries_fp8_n": (None, [P, P, P, i64, i32, i32, P]),
            "orc_mxfp4_encode_rows": (None, [P, i64, i32, P, P]),
            "orc_store_entries_nvfp4_n": (None, [P, i64, P, P]),
            "orc_load_entries_nvfp4_n": (None, [P, P, i64, P]),
            "orc_mxfp4_decode_rows": (None, [P, P, i64, i32, P]),
            "orc_compress": (i32, [P, P, P, P, P, P, P, i32, i64, i32, i32, i32, i32,
                                   i32, dbl, P, P]),
            "orc_rope": (None, [P, i32, i32, dbl, dbl]),
            "orc_index_scores": (None, [P, P, P, i32, i32, i32, i32, P]),
            "orc_topk": (None, [P, i32, i32, P]),
            "orc_index_topk_rows": (None, [P, P, P, i32, i32, i32, i32, i64, P, i32, i32,
                                           i32, P]),
            "orc_attend_rows": (i32, [P, i32, i32, i64, P, i32, i32, P, i32, i32, P, P, i64,
                                      i32, i32, P, i32, dbl, P, i32, P]),
            "orc_store_window_fp8_n": (None, [P, i64, i64, i32, dbl, P, P]),
            "orc_set_threads": (i32, [i32]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def set_threads(n):
    """Thread count of the row-parallel loops (timing only); returns the previous one."""
    return lib().orc_set_threads(int(n))


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ---- formats ----------------------------------------------------------------

def bf16_from_f32(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_bf16_from_f32_n(_p(x), x.size, _p(out))
    return out


def bf16_to_f64(b):
    b = _c(b, np.uint16)
    out = np.empty(b.shape, np.float64)
    lib().orc_bf16_to_f64_n(_p(b), b.size, _p(out))
    return out


def e4m3_from_f32(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().orc_e4m3_from_f32_n(_p(x), x.size, _p(out))
    return out


def e4m3_to_f32(c):
    c = _c(c, np.uint8)
    out = np.empty(c.shape, np.float32)
    lib().orc_e4m3_to_f32_n(_p(c), c.size, _p(out))
    return out


def mxfp4_encode(x):
    """x [..., n] (n % 32 == 0) -> (codes [..., n/2] u8, scales [..., n/32] u8)."""
    x = _c(x, np.float32)
    n = x.shape[-1]
    assert n % 32 == 0
    rows = x.size // n
    codes = np.empty(x.shape[:-1] + (n // 2,), np.uint8)
    scales = np.empty(x.shape[:-1] + (n // 32,), np.uint8)
    lib().orc_mxfp4_encode_rows(_p(x), rows, n, _p(codes), _p(scales))
    return codes, scales


def mxfp4_decode(codes, scales):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    n = codes.shape[-1] * 2
    rows = codes.size // (n // 2)
    out = np.empty(codes.shape[:-1] + (n,), np.float32)
    lib().orc_mxfp4_decode_rows(_p(codes), _p(scales), rows, n, _p(out))
    return out


def rope_rows_bf16(rows_bits, pos0, rope_dims=64, rope_base=10000.0):
    """Raw rows [n, 128] bf16 bits of positions pos0.. -> rows rotated at
    their positions (fp64), rounded to fp32 and then to bf16 (bits)."""
    r = bf16_to_f64(rows_bits)
    for i in range(r.shape[0]):
        lib().orc_rope(_p(r[i]), r.shape[1], rope_dims, float(rope_base), float(pos0 + i))
    return bf16_from_f32(r.astype(np.float32))


def store_window_fp8(win_bits, pos0, rope_dims=64, rope_base=10000.0):
    """Raw window rows [n, 128] bf16 bits of positions pos0.. -> the FP8
    window cache (codes [n, 128] e4m3 of the rotated rows, scale [n] f32)."""
    w = _c(win_bits, np.uint16)
    n = w.size // 128
    codes = np.empty(w.shape[:-1] + (128,), np.uint8)
    sc = np.empty(w.shape[:-1], np.float32)
    lib().orc_store_window_fp8_n(_p(w), n, int(pos0), rope_dims, float(rope_base), _p(codes), _p(sc))
    return codes, sc


def load_window_fp8(codes, scale):
    """FP8 window cache -> fp64 rows [n, 128] (code x scale, exact)."""
    codes = _c(codes, np.uint8)
    scale = _c(scale, np.float32)
    n = codes.size // 128
    out = np.empty(codes.shape[:-1] + (128,), np.float64)
    lib().orc_load_entries_fp8_n(_p(codes), None, _p(scale), n, 128, 0, _p(out))
    return out


def store_entries_nvfp4(rows_f32):
    """[n, 128] fp32 post-RoPE entries -> (records [n, 72] u8: e2m1 codes +
    e4m3 block scales, scale [n] f32)."""
    r = _c(rows_f32, np.float32)
    assert r.shape[-1] == 128
    n = r.size // 128
    recs = np.empty(r.shape[:-1] + (72,), np.uint8)
    sc = np.empty(r.shape[:-1], np.float32)
    lib().orc_store_entries_nvfp4_n(_p(r), n, _p(recs), _p(sc))
    return recs, sc


def load_entries_nvfp4(recs, scale):
    """NVFP4 records + scales -> fp64 rows [n, 128]."""
    recs = _c(recs, np.uint8)
    scale = _c(scale, np.float32)
    n = recs.size // 72
    out = np.empty(recs.shape[:-1] + (128,), np.float64)
    lib().orc_load_entries_nvfp4_n(_p(recs), _p(scale), n, _p(out))
    return out


def store_entries_fp8(rows_f32, rope_dims=64):
    """[n, D] fp32 -> (codes [n, D-R] u8, rope [n, R] bf16 bits, scale [n] f32)."""
    r = _c(rows_f32, np.float32)
    n, D = r.shape
    codes = np.empty((n, D - rope_dims), np.uint8)
    rope = np.empty((n, rope_dims), np.uint16)
    scale = np.empty((n,), np.float32)
    lib().orc_store_entries_fp8_n(_p(r), n, D, rope_dims, _p(codes), _p(rope), _p(scale))
    return codes, rope, scale


def load_entries_fp8(codes, rope, scale):
    codes = _c(codes, np.uint8)
    rope = _c(rope, np.uint16)
    scale = _c(scale, np.float32)
    n, nq = codes.shape
    R = rope.shape[1]
    out = np.empty((n, nq + R), np.float64)
    lib().orc_load_entries_fp8_n(_p(codes), _p(rope), _p(scale), n, nq + R, R, _p(out))
    return out


# ---- compression ------------------------------------------------------------

def compress(kv, beta, m, overlap, pos0=0, ik=None, z=None, prev_kv=None, prev_ik=None,
             prev_z=None, rope_dims=64, rope_base=10000.0):
    """One batch row.  kv [T, D] bf16 bits -> (entries [T//m, D] f32 post-RoPE,
    kidx [T//m, d_idx] f32 or None), both before storage rounding."""
    kv = _c(kv, np.uint16)
    T, D = kv.shape
    ik = _c(ik, np.uint16)
    d_idx = 0 if ik is None else ik.shape[1]
    beta = _c(beta, np.float32)
    z = _c(z, np.float32)
    prev_kv, prev_ik, prev_z = _c(prev_kv, np.uint16), _c(prev_ik, np.uint16), _c(prev_z, np.float32)
    n = T // m
    ent = np.empty((n, D), np.float32)
    kid = np.empty((n, d_idx), np.float32) if ik is not None else None
    r = lib().orc_compress(_p(kv), _p(ik), _p(z), _p(beta), _p(prev_kv), _p(prev_ik), _p(prev_z),
                           T, int(pos0), D, d_idx, m, int(overlap), rope_dims, float(rope_base),
                           _p(ent), _p(kid))
    if r < 0:
        raise ValueError("orc_compress rejected its arguments")
    return ent, kid


def rope(v, pos, rope_dims=64, rope_base=10000.0):
    v = np.array(v, dtype=np.float64, copy=True)
    lib().orc_rope(_p(v), v.shape[-1], rope_dims, float(rope_base), float(pos))
    return v


# ---- indexer / top-k --------------------------------------------------------

def index_scores(q_dec, w, keys_dec, relu=True):
    """q_dec [H_I, d], w [H_I], keys_dec [n_vis, d] (decoded values) -> [n_vis] f32."""
    q = _c(q_dec, np.float32)
    w = _c(w, np.float32)
    k = _c(keys_dec, np.float32)
    H_I, d = q.shape
    n = k.shape[0]
    out = np.empty((n,), np.float32)
    lib().orc_index_scores(_p(q), _p(w), _p(k), n, H_I, d, int(relu), _p(out))
    return out


def topk(scores, k):
    s = _c(scores, np.float32)
    out = np.empty((k,), np.int32)
    lib().orc_topk(_p(s), s.size, k, _p(out))
    return out


def index_topk_rows(q_dec, w, k_dec, m, q_pos0, rows, k, relu=True):
    """q_dec [n, H_I, d], w [n, H_I], k_dec [N, d]; rows: query row numbers."""
    q = _c(q_dec, np.float32)
    w = _c(w, np.float32)
    kk = _c(k_dec, np.float32)
    rows = _c(rows, np.int32)
    n, H_I, d = q.shape
    N = kk.shape[0]
    out = np.empty((rows.size, k), np.int32)
    lib().orc_index_topk_rows(_p(q), _p(w), _p(kk), H_I, d, N, m, int(q_pos0), _p(rows),
                              rows.size, k, int(relu), _p(out))
    return out


# ---- attention --------------------------------------------------------------

def attend_rows(q, q_pos0, entries_f64, m, rows, mode, idx=None, win=None, win_pos0=0,
                n_win=128, sink=None, rope_dims=64, rope_base=10000.0, win_post=None):
    """q [n, H, D] bf16 bits; entries_f64 [N, D] decoded post-RoPE entries;
    mode 'csa' (keys = idx rows) or 'hca' (keys = all visible entries);
    win [win_len, D] bf16 bits pre-RoPE starting at win_pos0, or win_post
    [win_len, D] fp64 rows already rotated (a decoded FP8 window cache).
    Returns out [len(rows), H, D] fp64."""
    q = _c(q, np.uint16)
    n, H, D = q.shape
    ent = _c(entries_f64, np.float64)
    if ent is None:
        ent = np.zeros((0, D), np.float64)
    N = ent.shape[0]
    rows = _c(rows, np.int32)
    idx = _c(idx, np.int32)
    k = 0 if idx is None else idx.shape[1]
    if mode == "csa":
        assert idx is not None and idx.shape[0] == rows.size
    win = _c(win, np.uint16)
    win_post = _c(win_post, np.float64)
    src = win if win_post is None else win_post
    win_len = 0 if src is None else src.shape[0]
    if src is None:
        n_win = 0
    sink = _c(sink, np.float32)
    out = np.empty((rows.size, H, D), np.float64)
    r = lib().orc_attend_rows(_p(q), H, D, int(q_pos0), _p(ent), N, m, _p(idx), k,
                              0 if mode == "csa" else 1, _p(win), _p(win_post), int(win_pos0), win_len,
                              int(n_win), _p(sink), rope_dims, float(rope_base), _p(rows),
                              rows.size, _p(out))
    if r != 0:
        raise ValueError("window source does not cover a needed row")
    return out
