"""Shared test utilities: host<->device marshalling, the oracle pipelines
(CPU, from oracle/), and the comparison rules.

Comparison rules
  * outputs: max-abs error <= 2e-2 and relative L1 (sum|gpu-ref| / sum|ref|)
    <= 5e-3 against the fp64 oracle;
  * MXFP4 top-k index sets: bit-exact;
  * bf16 top-k index sets: equal sizes, and every index in the symmetric
    difference has an oracle score within 1e-3 of the oracle's k-th score;
  * compressed entries and storage codes: bit-exact.
"""
from __future__ import annotations

import numpy as np
import torch

MAX_ABS = 2e-2
MEAN_REL = 5e-3
TIE_BAND = 1e-3


def dev(a, dtype=None):
    """numpy -> cuda tensor (uint16 arrays become bfloat16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    t = torch.from_numpy(a).cuda()
    return t if dtype is None else t.to(dtype)


def host_bits(t):
    """bfloat16 cuda tensor -> numpy uint16 bits."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t):
    return t.contiguous().cpu().numpy()


def bf16_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def out_errors(gpu_bits, ref):
    g = bf16_f64(gpu_bits)
    d = np.abs(g - ref)
    return float(d.max()), float(d.sum() / max(np.abs(ref).sum(), 1e-30))


def assert_close(gpu_bits, ref, what=""):
    mx, mr = out_errors(gpu_bits, ref)
    assert np.isfinite(mx), what
    assert mx <= MAX_ABS and mr <= MEAN_REL, "%s: max-abs %.3g (<= %g), mean-rel %.3g (<= %g)" % (
        what, mx, MAX_ABS, mr, MEAN_REL)
    return mx, mr


def canon_idx(rows):
    """Top-k rows as sets in the oracle's form: the selected indices
    ascending, then the -1 padding (the library's own order is checked
    separately by canonical_rows)."""
    rows = np.asarray(rows)
    out = np.full_like(rows, -1)
    for r in np.ndindex(rows.shape[:-1]):
        v = np.sort(rows[r][rows[r] >= 0])
        out[r][:v.size] = v
    return out


def canonical_rows(rows):
    """Top-k rows in the library's canonical order: the selected indices
    grouped by (index // 32) % 8, groups ascending, ascending within a group,
    then the -1 padding."""
    rows = np.asarray(rows)
    out = np.full_like(rows, -1)
    for r in np.ndindex(rows.shape[:-1]):
        v = rows[r][rows[r] >= 0].astype(np.int64)
        v = v[np.lexsort((v, (v >> 5) & 7))]
        out[r][:v.size] = v
    return out


def topk_tie_ok(got, ref, scores, nv, k):
    """bf16 rule: equal set sizes; the symmetric difference lies within
    TIE_BAND of the k-th largest oracle score.  Returns the number of rows
    that differ."""
    diff_rows = 0
    for r in range(got.shape[0]):
        a = set(int(x) for x in got[r] if x >= 0)
        b = set(int(x) for x in ref[r] if x >= 0)
        assert len(a) == len(b) == min(k, int(nv[r])), r
        v = got[r][got[r] >= 0]
        assert len(np.unique(v)) == v.size and (v.size == 0 or v.max() < int(nv[r])), "duplicate or invisible index"
        if a != b:
            diff_rows += 1
            sc = scores[r]
            kth = np.sort(sc[:int(nv[r])])[::-1][min(k, int(nv[r])) - 1]
            for s in a ^ b:
                assert abs(float(sc[s]) - float(kth)) <= TIE_BAND, (r, s, sc[s], kth)
    return diff_rows


# ---- oracle pipelines --------------------------------------------------------

def oracle_compress_store(orc, kv, beta, m, overlap, ik=None, z=None, pos0=0, prev_kv=None,
                          prev_ik=None, prev_z=None, kidx_fmt="mxfp4", entry_fmt="bf16"):
    """One batch row through the oracle compressor + storage encoders."""
    ent, kid = orc.compress(kv, beta, m, overlap, pos0=pos0, ik=ik, z=z, prev_kv=prev_kv,
                            prev_ik=prev_ik, prev_z=prev_z)
    res = {"entries_f32": ent, "kidx_f32": kid}
    if entry_fmt == "bf16":
        res["entries"] = orc.bf16_from_f32(ent)
        res["entries_f64"] = orc.bf16_to_f64(res["entries"])
    elif entry_fmt == "nvfp4":
        res["entries"], res["entry_scale"] = orc.store_entries_nvfp4(ent)
        res["entries_f64"] = orc.load_entries_nvfp4(res["entries"], res["entry_scale"])
    else:
        c, r, s = orc.store_entries_fp8(ent)
        res["entries"], res["entries_rope"], res["entry_scale"] = c, r, s
        res["entries_f64"] = orc.load_entries_fp8(c, r, s)
    if kid is not None:
        if kidx_fmt == "mxfp4":
            res["kidx"], res["kidx_scale"] = orc.mxfp4_encode(kid)
            res["kidx_dec"] = orc.mxfp4_decode(res["kidx"], res["kidx_scale"])
        else:
            res["kidx"] = orc.bf16_from_f32(kid)
            res["kidx_dec"] = orc.bf16_to_f64(res["kidx"]).astype(np.float32)
    return res


def oracle_q_dec(orc, q_bits, fmt):
    """Decoded indexer queries as the kernel sees them (bf16 values, or the
    MXFP4 encoding of the bf16 values)."""
    qf = orc.bf16_to_f64(q_bits).astype(np.float32)
    if fmt == "bf16":
        return qf
    c, s = orc.mxfp4_encode(qf)
    return orc.mxfp4_decode(c, s)
