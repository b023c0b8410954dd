"""C-ABI checks that need no GPU: the library loads, exports every function
include/csa.h declares, and rejects bad arguments on the host (status code +
csa_last_error message) before anything is launched.  Pointers passed here
are never dereferenced: every call fails validation first."""
import ctypes as C
import os
import re
import threading

import pytest

from long_context_attention_21_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # 16-byte aligned, never dereferenced
FAKE2 = 0x20000
MIS = 0x10008   # 8-byte aligned only


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from long_context_attention_21_amd import build
        build.build()
    return _lib.lib()


def _declared():
    src = open(os.path.join(ROOT, "include", "csa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", src, flags=re.M))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert {"csa_compress", "csa_index_topk", "csa_attend", "hca_attend"} <= names
    for n in names:
        assert hasattr(L, n), n
    assert set(_lib.EXPORTS) == names


def test_version(L):
    assert L.csa_version() >= 100


def _compress(L, **kw):
    a = dict(kv=FAKE, ik=None, z=None, beta=FAKE, prev_kv=None, prev_ik=None, prev_z=None, B=1,
             T=64, pos0=0, D=128, d_idx=64, m=4, overlap=1, rope_dims=64, rope_base=10000.0,
             entries_out=FAKE2, entries_rope_out=None, entry_scale_out=None, entry_fmt=0,
             kidx_out=None, kidx_scale_out=None, kidx_fmt=1, stream=None)
    a.update(kw)
    return L.csa_compress(*a.values())


def _msg(L):
    return L.csa_last_error().decode()


@pytest.mark.parametrize("kw,needle", [
    (dict(D=64), "D=64"),
    (dict(m=0), "m=0"),
    (dict(m=129), "m=129"),
    (dict(overlap=2), "overlap"),
    (dict(rope_dims=32), "rope_dims"),
    (dict(pos0=6), "pos0"),
    (dict(pos0=-4), "pos0"),
    (dict(beta=None), "beta"),
    (dict(kv=None), "kv is NULL"),
    (dict(entries_out=None), "entries_out"),
    (dict(entry_fmt=1), "entry_fmt"),
    (dict(entry_fmt=2), "FP8 entries"),
    (dict(pos0=8), "prev_kv"),
    (dict(pos0=8, prev_kv=FAKE, ik=FAKE), "prev_ik"),
    (dict(ik=FAKE, d_idx=32), "d_idx"),
    (dict(ik=FAKE, kidx_out=FAKE, kidx_fmt=1, kidx_scale_out=None), "kidx_scale_out"),
    (dict(ik=FAKE, kidx_out=FAKE, kidx_fmt=7), "kidx_fmt"),
    (dict(kv=FAKE + 2), "aligned"),
    (dict(B=-1), "B=-1"),
])
def test_compress_rejects(L, kw, needle):
    assert _compress(L, **kw) == _lib.CSA_INVALID_ARG
    assert needle in _msg(L)


def test_compress_empty_is_ok(L):
    assert _compress(L, T=3, kv=None, entries_out=None) == _lib.CSA_OK   # no complete block
    assert _compress(L, B=0) == _lib.CSA_OK
    assert _msg(L) == ""


def _index(L, **kw):
    a = dict(qidx=FAKE, qidx_scale=None, widx=FAKE, kidx=FAKE, kidx_scale=FAKE, fmt=1, B=1, n=16,
             q_pos0=0, H_I=8, d_idx=64, N=4, m=4, k=16, idx_out=FAKE2, ws=None, ws_bytes=0,
             fallback_count=None, stream=None)
    a.update(kw)
    return L.csa_index_topk(*a.values())


@pytest.mark.parametrize("kw,needle", [
    (dict(fmt=2), "fmt=2"),
    (dict(d_idx=128), "d_idx"),
    (dict(H_I=0), "H_I=0"),
    (dict(H_I=9), "H_I=9"),
    (dict(k=0), "k=0"),
    (dict(k=4096), "k=4096"),
    (dict(m=0), "m=0"),
    (dict(q_pos0=-1), "q_pos0"),
    (dict(qidx=None), "non-NULL"),
    (dict(idx_out=None), "non-NULL"),
    (dict(kidx=None), "kidx is NULL"),
    (dict(kidx_scale=None), "kidx_scale"),
    (dict(kidx=MIS), "aligned"),
    (dict(n=-1), "n=-1"),
    (dict(fallback_count=FAKE + 2), "fallback_count"),
])
def test_index_rejects(L, kw, needle):
    assert _index(L, **kw) == _lib.CSA_INVALID_ARG
    assert needle in _msg(L)


def test_index_workspace_query(L):
    assert L.csa_index_topk_workspace_bytes(1, 16, 0, 4, 4, 16) == 0
    # split path: few query rows over >= 65536 visible entries, one 32784-byte row each
    assert L.csa_index_topk_workspace_bytes(64, 1, 4 * 262144, 262144, 4, 2048) == 64 * 32784
    assert L.csa_index_topk_workspace_bytes(2, 4, 4 * 70000 - 4, 90000, 4, 2048) == 8 * 32784
    assert L.csa_index_topk_workspace_bytes(1, 5, 4 * 70000, 90000, 4, 2048) == 0     # too many rows
    assert L.csa_index_topk_workspace_bytes(64, 1, 4 * 60000, 262144, 4, 2048) == 0  # too few visible
    # the path depends on the rows of one batch entry, not on B
    assert L.csa_index_topk_workspace_bytes(600, 1, 4 * 262144, 262144, 4, 2048) == 600 * 32784


def test_index_rejects_small_or_misaligned_workspace(L):
    need = L.csa_index_topk_workspace_bytes(1, 1, 4 * 70000, 70000, 4, 512)
    base = dict(B=1, n=1, q_pos0=4 * 70000, N=70000, k=512)
    assert _index(L, **base, ws=FAKE, ws_bytes=need - 1) == _lib.CSA_WORKSPACE_TOO_SMALL
    assert _index(L, **base, ws=MIS, ws_bytes=need) == _lib.CSA_INVALID_ARG
    assert "ws must be" in _msg(L)
    assert _index(L, **base, ws=None, ws_bytes=need) == _lib.CSA_INVALID_ARG


def _attend(L, **kw):
    a = dict(q=FAKE, B=1, n=8, q_pos0=200, H=64, D=128, entries=FAKE, entries_rope=None,
             entry_scale=None, entry_fmt=0, N=50, m=4, idx=FAKE, k=16, win_kv=FAKE,
             win_pos0=73, win_len=200, n_win=128, win_fmt=0, win_scale=None, sink=None, rope_dims=64,
             rope_base=10000.0, out=FAKE2, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return L.csa_attend(*a.values())


@pytest.mark.parametrize("kw,needle", [
    (dict(D=64), "D=64"),
    (dict(H=0), "H=0"),
    (dict(H=65), "H=65"),
    (dict(m=0), "m=0"),
    (dict(entry_fmt=1), "entry_fmt"),
    (dict(entry_fmt=2), "FP8 entries"),
    (dict(rope_dims=16), "rope_dims"),
    (dict(n_win=-1), "n_win"),
    (dict(n_win=129), "n_win=129"),
    (dict(win_fmt=5, rope_dims=0), "pre-rotated window"),
    (dict(q=None), "non-NULL"),
    (dict(idx=None), "idx is NULL"),
    (dict(entries=None), "entries is NULL"),
    (dict(win_kv=None), "win_kv is NULL"),
    (dict(win_pos0=74), "does not cover"),       # needs position 200-127 = 73
    (dict(win_len=134), "does not cover"),       # needs up to 207
    (dict(q=MIS), "aligned"),
    (dict(q_pos0=-5), "q_pos0"),
    (dict(win_fmt=3), "win_fmt=3"),
    (dict(win_fmt=4, win_scale=FAKE), "FP8 or NVFP4 entries"),
    (dict(win_fmt=4, entry_fmt=2, entries_rope=FAKE, entry_scale=FAKE), "win_scale"),
])
def test_attend_rejects(L, kw, needle):
    assert _attend(L, **kw) == _lib.CSA_INVALID_ARG
    assert needle in _msg(L)


def test_hca_rejects(L):
    r = L.hca_attend(FAKE, 1, 8, 0, 64, 128, FAKE, 10, 0, FAKE, 0, 8, 128, 0, None, 64, 10000.0, FAKE2, None)
    assert r == _lib.CSA_INVALID_ARG and "m=0" in _msg(L)
    r = L.hca_attend(FAKE, 1, 8, 0, 64, 128, FAKE, 10, 4, FAKE, 0, 8, 128, 4, None, 64, 10000.0, FAKE2, None)
    assert r == _lib.CSA_INVALID_ARG and "win_fmt=4" in _msg(L)


@pytest.mark.parametrize("kw,needle", [
    (dict(rope_dims=0), "rope_dims=0"),
    (dict(T=-1), "T=-1"),
    (dict(out=None), "non-NULL"),
    (dict(kv=MIS + 2), "aligned"),
])
def test_rope_rows_rejects(L, kw, needle):
    a = dict(kv=FAKE, B=2, T=5, pos0=0, rope_dims=64, rope_base=10000.0, out=FAKE2, stream=None)
    a.update(kw)
    assert L.csa_rope_rows(*a.values()) == _lib.CSA_INVALID_ARG
    assert needle in _msg(L)


def test_last_error_is_thread_local(L):
    assert _attend(L, D=64) == _lib.CSA_INVALID_ARG
    seen = {}

    def other():
        seen["before"] = _msg(L)
        _index(L, k=0)
        seen["after"] = _msg(L)

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["before"] == ""
    assert "k=0" in seen["after"]
    assert "D=64" in _msg(L)


def test_binding_has_no_fallback(monkeypatch, tmp_path):
    """The Python binding raises when the library is missing (no CPU path)."""
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()


def _append(L, **kw):
    a = dict(kv_new=FAKE, ik_new=None, z_new=None, B=2, t=3, kv_ring=FAKE2, ik_ring=None, z_ring=None,
             win8_ring=None, win8_scale=None, W=128, beta=FAKE, m=4, overlap=1, rope_dims=64, rope_base=10000.0, entries=FAKE,
             entries_rope=None, entry_scale=None, entry_fmt=0, kidx=None, kidx_scale=None, kidx_fmt=1,
             N_cap=8, stream=None)
    a.update(kw)
    return L.csa_cache_append(*a.values())


@pytest.mark.parametrize("kw,needle", [
    (dict(W=7), "W=7"),                       # the 2m = 8 pooled rows do not fit the ring
    (dict(N_cap=0), "does not fit"),          # t = 3 completes entry 0
    (dict(ik_new=FAKE), "ik_new and ik_ring"),
    (dict(z_ring=FAKE), "z_new and z_ring"),
    (dict(entries=None), "entries is NULL"),
    (dict(t=-1), "t must be"),
    (dict(entry_fmt=1), "entry_fmt=1"),
    (dict(kv_ring=MIS + 2), "aligned"),
    (dict(win8_ring=FAKE), "win8_ring and win8_scale"),
])
def test_cache_append_rejects(L, kw, needle):
    assert _append(L, **kw) == _lib.CSA_INVALID_ARG
    assert needle in _msg(L)


def test_cache_append_needs_no_cache_between_blocks(L):
    # t = 4 completes no block (m = 4): caches may be NULL.  Validation only:
    # B = 0 launches nothing.
    assert _append(L, B=0, t=4, entries=None) == _lib.CSA_OK


def test_attend_workspace_query(L):
    # bf16 entries never split; FP8 and NVFP4 entries with >= 16 chunks do,
    # whatever B and n are (tokens run in blocks of at most 512)
    assert L.csa_attend_workspace_bytes(64, 1, 2048, 128, 0) == 0
    assert L.csa_attend_workspace_bytes(64, 1, 2048, 128, 2) == 64 * 9 * 33280
    assert L.csa_attend_workspace_bytes(64, 1, 512, 128, 2) == 64 * 3 * 33280  # 20 chunks
    assert L.csa_attend_workspace_bytes(64, 1, 64, 128, 2) == 0       # 6 chunks: one work-group
    assert L.csa_attend_workspace_bytes(600, 1, 2048, 128, 2) == 512 * 9 * 33280
    assert L.csa_attend_workspace_bytes(2, 4096, 2048, 128, 3) == 512 * 9 * 33280


def test_attend_rejects_small_workspace(L):
    kw = dict(B=2, n=1, q_pos0=4000, N=1000, k=2048, entry_fmt=2, entries_rope=FAKE, entry_scale=FAKE,
              win_pos0=3873, win_len=128)
    need = L.csa_attend_workspace_bytes(2, 1, 2048, 128, 2)
    assert _attend(L, **kw, ws=FAKE, ws_bytes=need - 16) == _lib.CSA_WORKSPACE_TOO_SMALL
    assert _attend(L, **kw, ws=None, ws_bytes=need) == _lib.CSA_INVALID_ARG
    assert "ws must be" in _msg(L)


_EVS = (C.c_void_p * 3)(FAKE, FAKE2, MIS)  # never recorded: every call below fails validation first


def _index_attend(L, **kw):
    a = dict(qidx=FAKE, qidx_scale=None, widx=FAKE, kidx=FAKE, kidx_scale=FAKE, kidx_fmt=1, H_I=8, d_idx=64,
             k=64, idx_out=FAKE2, fallback_count=None, q=FAKE, H=64, D=128, entries=FAKE, entries_rope=None,
             entry_scale=None, entry_fmt=0, win_kv=FAKE, win_pos0=0, win_len=4096, n_win=128, win_fmt=5,
             win_scale=None, sink=None, rope_dims=64, rope_base=10000.0, out=FAKE2, B=1, n=4096, q_pos0=0,
             N=1024, m=4, n_chunks=4, stream=None, aux_stream=FAKE, events=_EVS)
    a.update(kw)
    return L.csa_index_attend(*a.values())


@pytest.mark.parametrize("kw,needle,status", [
    (dict(n_chunks=0), "n_chunks=0", _lib.CSA_INVALID_ARG),
    (dict(entry_fmt=7), "entry_fmt=7", _lib.CSA_INVALID_ARG),
    (dict(aux_stream=None), "aux_stream", _lib.CSA_INVALID_ARG),
    (dict(events=None), "three events", _lib.CSA_INVALID_ARG),
    (dict(events=(C.c_void_p * 3)(FAKE, None, FAKE)), "three events", _lib.CSA_INVALID_ARG),
    (dict(events=(C.c_void_p * 3)(FAKE, FAKE2, FAKE)), "distinct", _lib.CSA_INVALID_ARG),
    # the indexer's and the attention's own checks, before anything is enqueued
    (dict(k=0), "k=0", _lib.CSA_INVALID_ARG),
    (dict(H_I=9), "H_I=9", _lib.CSA_INVALID_ARG),
    (dict(n_win=129), "n_win=129", _lib.CSA_INVALID_ARG),
    (dict(win_len=100), "window source", _lib.CSA_INVALID_ARG),
    (dict(q=MIS), "aligned", _lib.CSA_INVALID_ARG),
    # B > 1 or fewer than 1024 tokens run as one chunk: no aux stream or
    # events are asked for, the later checks still apply
    (dict(B=2, aux_stream=None, events=None, k=0), "k=0", _lib.CSA_INVALID_ARG),
    (dict(n=1000, aux_stream=None, events=None, k=0), "k=0", _lib.CSA_INVALID_ARG),
    # calls that would need a workspace are refused (decode shapes)
    (dict(n=4, q_pos0=4 * 65536, N=65536, win_pos0=4 * 65536 - 127, win_len=131), "workspace",
     _lib.CSA_WORKSPACE_TOO_SMALL),
    (dict(n=1, q_pos0=8000, N=2000, k=2048, entry_fmt=2, entries_rope=FAKE, entry_scale=FAKE, win_fmt=0,
          win_pos0=7873, win_len=128), "workspace", _lib.CSA_WORKSPACE_TOO_SMALL),
])
def test_index_attend_rejects(L, kw, needle, status):
    assert _index_attend(L, **kw) == status
    assert needle in _msg(L), _msg(L)


def _proj_in(L, **kw):
    a = dict(x=FAKE, M=5, d=256, w_in=FAKE2, n_q=512, n_kv=128, n_ik=64, n_lat=32, n_w=8, n_z=2, w_up=FAKE,
             n_qidx=512, q_out=FAKE, kv_out=FAKE, ik_out=FAKE, lat_out=FAKE, w_out=FAKE, z_out=FAKE, qidx_out=FAKE,
             qidx_scale_out=FAKE2, stream=None)
    a.update(kw)
    return L.csa_project_in(*a.values())


@pytest.mark.parametrize("kw,needle", [
    (dict(d=100), "d=100"),
    (dict(n_q=0, n_kv=0, n_ik=0, n_lat=0, n_w=0, n_z=0, n_qidx=0), "no output"),
    (dict(z_out=None), "z_out is NULL"),
    (dict(n_q=1 << 30), "too large"),
    (dict(kv_out=None), "kv_out is NULL"),
    (dict(x=MIS), "aligned"),
    (dict(n_lat=0), "needs the latent"),
    (dict(n_lat=24), "rank r=24"),
    (dict(n_qidx=48), "n_qidx=48"),
    (dict(n_qidx=-32), "n_qidx=-32"),
    (dict(qidx_scale_out=None), "non-NULL"),
    (dict(M=-1), "M=-1"),
    (dict(M=1 << 20, d=1024), "2 GiB"),
])
def test_project_in_rejects(L, kw, needle):
    assert _proj_in(L, **kw) == _lib.CSA_INVALID_ARG
    assert needle in _msg(L)


def test_project_in_empty_is_ok(L):
    assert _proj_in(L, M=0) == _lib.CSA_OK


@pytest.mark.parametrize("kw,needle", [
    (dict(r=8), "rank r=8"),
    (dict(lat=MIS), "latent"),
    (dict(q_f32_out=MIS), "aligned"),
    (dict(w_up=None), "non-NULL"),
])
def test_project_qidx_rejects(L, kw, needle):
    a = dict(lat=FAKE, M=3, r=32, w_up=FAKE2, n_qidx=512, qidx_out=FAKE, qidx_scale_out=FAKE, q_f32_out=None,
             stream=None)
    a.update(kw)
    assert L.csa_project_qidx(*a.values()) == _lib.CSA_INVALID_ARG
    assert needle in _msg(L)


@pytest.mark.parametrize("kw,needle", [
    (dict(G=3), "multiple of G=3"),
    (dict(D=100, H=1, G=1), "multiple of 32"),
    (dict(d=102), "d=102"),
    (dict(y_out=None), "non-NULL"),
    (dict(o=MIS), "aligned"),
])
def test_project_out_rejects(L, kw, needle):
    a = dict(o=FAKE, M=4, H=8, D=128, G=4, w_o=FAKE2, d=256, y_out=FAKE, stream=None)
    a.update(kw)
    assert L.csa_project_out(*a.values()) == _lib.CSA_INVALID_ARG
    assert needle in _msg(L)


def test_binding_checks_the_entry_row_width():
    """FP8 entries passed without entries_rope would read as NVFP4 records:
    the binding refuses rows of the wrong width before calling the library."""
    torch = pytest.importorskip("torch")
    import long_context_attention_21_amd as Lb
    q = torch.zeros((1, 1, 8, 128), dtype=torch.bfloat16)
    ent = torch.zeros((1, 16, 64), dtype=torch.uint8)
    with pytest.raises(ValueError, match="nvfp4"):
        Lb.csa_attend(q, ent, torch.zeros((1, 1, 4), dtype=torch.int32), entry_scale=torch.zeros((1, 16)))


def _index_noalloc(L, **kw):
    a = dict(qidx=FAKE, qidx_scale=None, widx=FAKE, kidx=FAKE, kidx_scale=FAKE, fmt=1, B=1, n=16,
             q_pos0=0, H_I=8, d_idx=64, N=4, m=4, k=16, idx_out=FAKE2, fallback_count=None, stream=None)
    a.update(kw)
    return L.csa_index_topk_noalloc(*a.values())


def test_index_noalloc_rejects_beyond_the_static_scratch(L):
    """257 split rows need more than the 8 MiB static scratch: rejected on the
    host, before any device call; bad arguments are rejected as by
    csa_index_topk."""
    assert L.csa_index_topk_workspace_bytes(257, 1, 4 * 70000, 70000, 4, 2048) == 257 * 32784
    r = _index_noalloc(L, B=257, n=1, q_pos0=4 * 70000, N=70000, k=2048)
    assert r == _lib.CSA_WORKSPACE_TOO_SMALL
    assert "static scratch" in _msg(L) and "csa_index_topk_noalloc" in _msg(L)
    assert _index_noalloc(L, k=0) == _lib.CSA_INVALID_ARG and "k=0" in _msg(L)
    assert _index_noalloc(L, kidx=MIS) == _lib.CSA_INVALID_ARG
    assert _index_noalloc(L, B=0) == _lib.CSA_OK
