"""Benchmark of the hybrid compressed attention forward on one MI355X.

Default workload (the 128K-context configuration): one CSA layer prefill,
batch 1, 131072 query tokens, 64 heads of dim 128 with RoPE on the last 64
dims, m = 4 overlapped compression (32768 entries), MXFP4 Lightning Indexer
(8 heads x 64, q quantised in-kernel), top-k 2048, 128-token window, per-head
sink.  One step = csa_compress -> csa_rope_rows (the window rotated once) ->
csa_index_attend over the whole sequence, inputs resident in HBM:
csa_index_topk and csa_attend pipelined over 16 token chunks, the indexer of
chunk c + 1 on a second stream beside the attention of chunk c (--chunks 1:
the calls in turn).

The default run also times, with the same steps, the two HBM-bound
workloads and reports each under "workloads" with its own roofline and
oracle baseline: the HCA layer forward (32768 tokens, m' = 128) and the CSA
decode step (64 sequences at t = 1M).  --config N times one workload alone
(1: the small CSA layer, 2: HCA, 3: the default, 4: decode, 5: the chunked
prefill of a CSA + HCA layer pair).

Prints one JSON line: throughput (query tokens/s), the roofline of the
dominant kernel (per-kernel durations from HIP events recorded on the launch
stream over the timed region; for a pipelined step, over a second pass of
the same steps with the calls in turn), per-kernel figures, and the CPU oracle timed
on a bounded sample of the same workload with all host cores and with one
thread (N = 1 only); a rate scaled up from a row sample says
"extrapolated".
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA/HCA forward query-tokens/s at 128K ctx; % MFMA / HBM roofline"
PEAK = {"bf16": 2500.0, "fp4": 10100.0, "hbm": 8000.0}  # TFLOP/s, TFLOP/s, GB/s (MI355X)

# HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
# (scaled by the plain-copy calibration of --copy-probe; a call of several
# kernels sums them), keyed by the sha256 of the kernel source they were
# taken on: a changed kernel reports null until it is measured again.  The
# summaries are profiles/<workload>_hbm_counters.txt.
TRAFFIC = {
    ('csa_attend', 3): {"sha256": "71df24787571677521eb64a0726bef4b05a552d4332d9a05f3b449d45ed08d4b", "bytes": 1.941e+10},  # csa_prefill_128k
    ('csa_index_topk', 3): {"sha256": "1ebf0f2e46b7587dddc74f1ad9e5325151889e29d886181e441c7940a1bdd024", "bytes": 1.222e+09},  # csa_prefill_128k
    ('csa_compress', 3): {"sha256": "9def0ef3ce63aa439bf0cab9ffe57b6148e0da778a945889a248fd9cdfded242", "bytes": 7.299e+07},  # csa_prefill_128k
    ('csa_rope_rows', 3): {"sha256": "9def0ef3ce63aa439bf0cab9ffe57b6148e0da778a945889a248fd9cdfded242", "bytes": 6.719e+07},  # csa_prefill_128k
    ('hca_attend', 2): {"sha256": "71df24787571677521eb64a0726bef4b05a552d4332d9a05f3b449d45ed08d4b", "bytes": 1.142e+09},  # hca_32k
    ('csa_compress', 2): {"sha256": "9def0ef3ce63aa439bf0cab9ffe57b6148e0da778a945889a248fd9cdfded242", "bytes": 8.835e+06},  # hca_32k
    ('csa_rope_rows', 2): {"sha256": "9def0ef3ce63aa439bf0cab9ffe57b6148e0da778a945889a248fd9cdfded242", "bytes": 1.685e+07},  # hca_32k
    ('csa_index_topk', 4): {"sha256": "1ebf0f2e46b7587dddc74f1ad9e5325151889e29d886181e441c7940a1bdd024", "bytes": 6.095e+08},  # csa_decode_1m
    ('csa_attend', 4): {"sha256": "71df24787571677521eb64a0726bef4b05a552d4332d9a05f3b449d45ed08d4b", "bytes": 1.038e+08},  # csa_decode_1m
}
TRAFFIC[("csa_project_in", "proj")] = {  # the GEMM (1.085e9) + the indexer-query kernel (9.7e6)
    "sha256": "59d66afdeef9ae5420b43f5642fb7e92fad86f487007ac22a01617daafc9a5f5", "bytes": 1.095e9}
KERNEL_SOURCE = {"csa_compress": "compress.hip", "hca_compress": "compress.hip", "csa_index_topk": "index_topk.hip",
                 "csa_attend": "attend.hip", "hca_attend": "attend.hip", "csa_project_in": "proj.hip",
                 "csa_rope_rows": "compress.hip", "hca_rope_rows": "compress.hip",
                 "csa_project_out": "proj.hip"}


def source_sha(kernel):
    import hashlib
    path = os.path.join(ROOT, "long_context_attention_21_amd", "csrc", KERNEL_SOURCE[kernel])
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_bytes(kernel, config):
    t = TRAFFIC.get((kernel, config))
    if t is None or t["sha256"] != source_sha(kernel):
        return None
    return t["bytes"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=None, choices=[1, 2, 3, 4, 5],
                    help="time this workload alone (default: config 3, with configs 2 and 4 beside it "
                         "under 'workloads')")
    ap.add_argument("--no-extra", action="store_true", help="default run: leave out configs 2 and 4")
    ap.add_argument("--chunks", type=int, default=None,
                    help="configs 1, 3 and 5: token chunks of csa_index_attend (the indexer of a chunk runs on a "
                         "second stream beside the attention of the chunk before; default min(16, tokens / 8192), config 5: 1); "
                         "1 = the two calls in turn")
    ap.add_argument("--trace-summary", default=None, metavar="CSV",
                    help="only summarise a rocprofv3 kernel_trace.csv (dispatches, total and average duration "
                         "per kernel and grid size) or counter_collection.csv (mean counter values per dispatch)")
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="query rows (config 4: sequences) of the oracle sample (default per config)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only copy 1 GiB device-to-device 3 times (HBM counter calibration)")
    ap.add_argument("--print-sha", action="store_true", help="print the kernel source hashes and exit")
    ap.add_argument("--append-probe", action="store_true",
                    help="only time the decode cache write path (csa_cache_append), 64 sequences at 1M")
    ap.add_argument("--entry-fmt", default="fp8", choices=["fp8", "nvfp4"],
                    help="config 4 only: the decode cache's entry format (fp8: e4m3 + bf16 RoPE dims; nvfp4: "
                         "the V4.1 variant, post-RoPE NVFP4)")
    ap.add_argument("--proj-probe", action="store_true",
                    help="only time the projections around the path (csa_project_in with the indexer "
                         "query, csa_project_out) at the prefill chunk shape")
    return ap.parse_args()


def proj_probe(steps=20, no_cpu=False):
    """The projections around the attention path for one prefill chunk of
    8192 tokens: hidden 4096 -> 64 query heads of 128, the shared KV row
    (128), the indexer key stream (64), a rank-32 indexer latent, 8 indexer
    head weights and 2 compression logits in one GEMM, then the MXFP4
    indexer query (8 heads of 64); out: the grouped output projection
    (8 groups of 8 heads) back to 4096.  Random-init bf16 weights."""
    import torch
    import long_context_attention_21_amd as L
    M, d, H, H_I, r, G = 8192, 4096, 64, 8, 32, 8
    widths = (H * 128, 128, 64, r, H_I, 2)
    g = torch.Generator(device="cuda").manual_seed(6)
    x = torch.randn((M, d), generator=g, device="cuda").to(torch.bfloat16)
    w_in = (torch.randn((sum(widths), d), generator=g, device="cuda") * d ** -0.5).to(torch.bfloat16)
    w_up = (torch.randn((H_I * 64, r), generator=g, device="cuda") * r ** -0.5).to(torch.bfloat16)
    KG = H // G * 128
    o = torch.randn((M, H, 128), generator=g, device="cuda").to(torch.bfloat16)
    w_o = (torch.randn((d, KG), generator=g, device="cuda") * KG ** -0.5).to(torch.bfloat16)
    outs = L.csa_project_in(x, w_in, widths, w_up=w_up, n_qidx=H_I * 64)
    y = L.csa_project_out(o, w_o, G)
    calls = {"csa_project_in": (lambda: L.csa_project_in(x, w_in, widths, w_up=w_up, n_qidx=H_I * 64, out=outs),
                                2.0 * M * sum(widths) * d + 2.0 * M * H_I * 64 * r),
             "csa_project_out": (lambda: L.csa_project_out(o, w_o, G, out=y), 2.0 * M * d * KG)}
    res = {}
    for name, (fn, flops) in calls.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        tf = flops / (ms / 1e3) / 1e12
        res[name] = {"ms": round(ms, 4), "flops": flops, "achieved": round(tf, 1), "peak": PEAK["bf16"],
                     "unit": "TFLOP/s", "frac": round(tf / PEAK["bf16"], 4)}
    ms_total = sum(r["ms"] for r in res.values())
    dom = res["csa_project_in"]
    cpu = None
    if not no_cpu:
        cpu = proj_cpu_baseline(d, H, H_I, r, G, widths)
    print(json.dumps({
        "metric": "projections around the attention path: tokens/s (input projections + indexer query + "
                  "grouped output projection)",
        "value": round(M / (ms_total / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "ms_per_step": round(ms_total, 4), "higher_is_better": True, "dtype": "bf16 (MFMA, fp32 accumulation)",
        "data": "synthetic (seeded torch.randn, random-init weights)",
        "config": {"workload": "projections of one 8192-token prefill chunk: hidden 4096, 64 query heads, "
                               "rank-32 MXFP4 indexer query (8 heads), 8 output groups", "tokens": M, "hidden": d},
        "roofline": {"kernel": "csa_project_in", "bound": "mfma", "achieved": dom["achieved"], "peak": dom["peak"],
                     "unit": "TFLOP/s", "frac": dom["frac"], "traffic": traffic_bytes("csa_project_in", "proj")},
        "kernels": res, "cpu_baseline": cpu}), flush=True)


def proj_cpu_baseline(d, H, H_I, r, G, widths, rows=8192, chunks=4):
    """The projection oracle (numpy fp64) on `chunks` chunks of `rows` tokens
    with full-size weights, scaled to tokens/s."""
    import oracle
    from oracle import projections as P
    rng = np.random.default_rng(0)

    def w(shape, scale):
        return oracle.bf16_from_f32((rng.standard_normal(shape) * scale).astype(np.float32))
    Ws = [w((n, d), d ** -0.5) for n in widths]
    w_up = w((H_I * 64, r), r ** -0.5)
    KG = H // G * 128
    w_o = w((d, KG), KG ** -0.5)
    t = 0.0
    for _ in range(chunks):
        x = w((rows, d), 1.0)
        o = w((rows, H * 128), 1.0)
        t0 = time.time()
        P.project_in(x, Ws[0], Ws[1], Ws[2], Ws[3], Ws[4], w_up, w_z=Ws[5])
        P.project_out(o, w_o, G)
        t += time.time() - t0
    return {"value": round(chunks * rows / t, 1), "unit": "tokens/s", "cores": _cores(), "kind": "oracle",
            "sample": "%d chunks of %d tokens through the projection oracle (input projections, indexer query, "
                      "grouped output projection) with full-size weights, %.1f s" % (chunks, rows, t)}


def _cores():
    cores = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    return min(cores, int(omp)) if omp else cores


def copy_probe():
    """A plain copy of known size: 1 GiB read + 1 GiB written per launch."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": src.numel() * 4, "copy_probe_bytes_written": dst.numel() * 4,
                      "launches": 3}), flush=True)


def append_probe(steps=1024, no_cpu=False):
    """The decode cache write path at config 4's shape: 64 sequences append
    one token per call at positions 1,048,576 .. +steps-1, into a CSA layer
    (m = 4 overlapped, FP8 + bf16-RoPE entries, MXFP4 indexer keys) and an
    HCA layer (m' = 128, bf16 entries), each with a 128-row state ring.
    Inputs are synthetic (ring contents do not affect the work)."""
    import torch
    import long_context_attention_21_amd as L
    B, P, W = 64, 1 << 20, 128
    cu = "cuda"
    g = torch.Generator(device=cu).manual_seed(5)
    kv = (torch.randn((steps, B, 128), generator=g, device=cu) * 0.1).to(torch.bfloat16)
    ik = (torch.randn((steps, B, 64), generator=g, device=cu) * 0.1).to(torch.bfloat16)
    res = {}
    for name, m, ov, efmt, with_ik in (("csa", 4, 1, "fp8", True), ("hca", 128, 0, "bf16", False)):
        N_cap = (P + steps) // m
        beta = torch.randn((2 * m if ov else m,), generator=g, device=cu)
        ring = (torch.randn((B, 2 * W, 128), generator=g, device=cu) * 0.1).to(torch.bfloat16)
        ik_ring = (torch.randn((B, W, 64), generator=g, device=cu) * 0.1).to(torch.bfloat16) if with_ik else None
        caches = {}
        if efmt == "bf16":
            caches["entries"] = torch.empty((B, N_cap, 128), dtype=torch.bfloat16, device=cu)
        else:
            caches["entries"] = torch.empty((B, N_cap, 64), dtype=torch.uint8, device=cu)
            caches["entries_rope"] = torch.empty((B, N_cap, 64), dtype=torch.bfloat16, device=cu)
            caches["entry_scale"] = torch.empty((B, N_cap), dtype=torch.float32, device=cu)
        if with_ik:
            caches["kidx"] = torch.empty((B, N_cap, 32), dtype=torch.uint8, device=cu)
            caches["kidx_scale"] = torch.empty((B, N_cap, 2), dtype=torch.uint8, device=cu)

        def call(i):
            L.csa_cache_append(kv[i], beta, m, ov, P + i, ring, caches, ik_new=ik[i] if with_ik else None,
                               ik_ring=ik_ring, entry_fmt=efmt, kidx_fmt="mxfp4")
        for i in range(8):
            call(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            call(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        Lr = 2 * m if ov else m
        row_in = 256 + (128 if with_ik else 0)
        entry_out = (196 if efmt == "fp8" else 256) + (34 if with_ik else 0)
        per_call = B * ((2 * 256 + (128 if with_ik else 0)) + (Lr * row_in + entry_out) / m)
        res[name] = {"us_per_call": round(us, 3), "tokens_per_s": round(B / us * 1e6, 1),
                     "algorithmic_bytes_per_call": int(per_call), "achieved_GBps": round(per_call / us * 1e-3, 2)}
    tot_us = sum(r["us_per_call"] for r in res.values())
    tot_bytes = sum(r["algorithmic_bytes_per_call"] for r in res.values())
    dom = max(res, key=lambda k: res[k]["us_per_call"])
    print(json.dumps({
        "metric": "decode cache write path: appended tokens/s (CSA + HCA layer per token)",
        "value": round(B / tot_us * 1e6, 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "ms_per_step": round(tot_us / 1e3, 5), "higher_is_better": True, "dtype": "fp32 pooling; fp8/bf16/mxfp4 storage",
        "data": "synthetic (seeded torch.randn)",
        "config": {"workload": "64 sequences append one token at positions 1048576.. into a CSA (m=4 overlapped, "
                               "FP8 + bf16-RoPE entries, MXFP4 keys) and an HCA (m'=128, bf16) layer",
                   "sequences": B, "q_pos": P},
        "roofline": {"kernel": "compress_kernel (append, %s)" % dom, "bound": "hbm",
                     "achieved": res[dom]["achieved_GBps"], "peak": PEAK["hbm"], "unit": "GB/s",
                     "frac": round(res[dom]["achieved_GBps"] / PEAK["hbm"], 5), "traffic": None},
        "append_probe": res, "algorithmic_bytes_per_step": tot_bytes,
        "cpu_baseline": None if no_cpu else append_cpu_baseline()}), flush=True)


def append_cpu_baseline(seqs=64, T=32768):
    """The compression oracle with the storage encoders over `seqs`
    sequences of T tokens for both layers, scaled to appended tokens/s."""
    import oracle
    rng = np.random.default_rng(0)
    t0 = time.time()
    for _ in range(seqs):
        kv = oracle.bf16_from_f32((rng.standard_normal((T, 128)) * 0.1).astype(np.float32))
        ik = oracle.bf16_from_f32((rng.standard_normal((T, 64)) * 0.1).astype(np.float32))
        ent, kid = oracle.compress(kv, rng.standard_normal(8).astype(np.float32), 4, 1, ik=ik)
        oracle.store_entries_fp8(ent)
        oracle.mxfp4_encode(kid)
        ent, _ = oracle.compress(kv, rng.standard_normal(128).astype(np.float32), 128, 0)
        oracle.bf16_from_f32(ent)
    t = time.time() - t0
    return {"value": round(seqs * T / t, 1), "unit": "tokens/s", "cores": _cores(), "kind": "oracle",
            "sample": "%d sequences x %d tokens through the compression oracle and storage encoders, "
                      "CSA and HCA layer, %.2f s" % (seqs, T, t)}


# ---------------------------------------------------------------- workloads --

def dev_bf16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def beside(side, first, second):
    """Run first() on a side stream beside second() on the current stream,
    then make the current stream wait for both: the two are independent
    calls of one layer step (the window rotation and the compression both
    only read the layer's KV rows)."""
    import torch
    cur = torch.cuda.current_stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        first()
    second()
    cur.wait_stream(side)


class CsaLayer:
    """Config 1 / 3: csa_compress -> csa_index_topk -> csa_attend."""

    def __init__(self, cfg_id):
        import torch
        import long_context_attention_21_amd as L
        from long_context_attention_21_amd import synth
        t0 = time.time()
        self.c = c = synth.config(cfg_id)
        log("inputs generated in %.1f s" % (time.time() - t0))
        self.L = L
        self.n, self.H, self.k, self.m = c["n"], c["H"], c["k"], c["m"]
        self.fmt = c["indexer"]
        self.q, self.kv, self.ik = dev_bf16(c["q"]), dev_bf16(c["kv"]), dev_bf16(c["ik"])
        self.qI, self.w = dev_bf16(c["q_I"]), dev(c["w_I"])
        self.beta, self.sink = dev(c["beta"]), dev(c["sink"])
        n, N = self.n, self.n // self.m
        self.N = N
        kshape = (1, N, 32) if self.fmt == "mxfp4" else (1, N, 64)
        kdt = torch.uint8 if self.fmt == "mxfp4" else torch.bfloat16
        self.bufs = {"entries": torch.empty((1, N, 128), dtype=torch.bfloat16, device="cuda"),
                     "kidx": torch.empty(kshape, dtype=kdt, device="cuda")}
        if self.fmt == "mxfp4":
            self.bufs["kidx_scale"] = torch.empty((1, N, 2), dtype=torch.uint8, device="cuda")
        self.idx = torch.empty((1, n, self.k), dtype=torch.int32, device="cuda")
        self.out = torch.empty((1, n, self.H, 128), dtype=torch.bfloat16, device="cuda")
        self.fallbacks = torch.zeros(1, dtype=torch.int32, device="cuda")  # exact-path work-groups
        self.kernels = ["csa_compress", "csa_rope_rows", "csa_index_topk", "csa_attend"]
        self.kv_rot = torch.empty_like(self.kv)
        # algorithmic work: indexer pairs (query, visible entry) and attention keys
        t = np.arange(n, dtype=np.int64)
        nv = np.minimum(N, (t + 1) // self.m)
        pairs = int(nv.sum())
        keys = int((np.minimum(self.k, nv) + np.minimum(t + 1, 128)).sum())
        kbytes = 34 if self.fmt == "mxfp4" else 128
        self.work = {
            "csa_compress": ("hbm", n * (256 + 128) + N * (256 + kbytes)),
            "csa_rope_rows": ("hbm", n * 512),
            "csa_index_topk": ("fp4" if self.fmt == "mxfp4" else "bf16", 2.0 * 8 * 64 * pairs
                               if self.fmt == "mxfp4" else 2.0 * c["H_I"] * 64 * pairs),
            "csa_attend": ("bf16", 4.0 * self.H * 128 * keys),
        }
        self.pairs, self.keys = pairs, keys
        self.calls = 0
        self.side = torch.cuda.Stream()
        if self.chunks is None:
            self.chunks = max(1, min(16, n // 8192))

    # csa_index_attend's token chunks in the timed step (1: the calls in
    # turn); None: 16, or fewer so that a chunk holds at least 8192 tokens
    # (small layers gain nothing from the second stream: config 1, 1024
    # tokens, took 0.186 ms/step in 2 chunks against 0.069 ms in turn)
    chunks = None

    def step(self, ev=None, serial=False):
        """One layer step.  With per-kernel events (or serial) the four calls
        run in turn on the current stream; otherwise the window rotation runs
        on a side stream beside the compression, and the indexer and the
        attention run as csa_index_attend over self.chunks token chunks."""
        L = self.L
        self.calls += 1
        compress = lambda: L.csa_compress(self.kv, self.beta, self.m, 1, ik=self.ik, kidx_fmt=self.fmt,
                                          out=self.bufs)
        rope = lambda: L.csa_rope_rows(self.kv, out=self.kv_rot)
        if ev is None and not serial and self.chunks > 1:
            beside(self.side, rope, compress)
            L.csa_index_attend(self.qI, self.w, self.bufs["kidx"], self.k, self.m, self.q, self.bufs["entries"],
                               fmt=self.fmt, kidx_scale=self.bufs.get("kidx_scale"), idx_out=self.idx,
                               fallback_count=self.fallbacks, win_kv=self.kv_rot, win_roped=True, sink=self.sink,
                               out=self.out, n_chunks=self.chunks)
            return
        if ev: ev[0].record()
        compress()
        if ev: ev[1].record()
        rope()
        if ev: ev[2].record()
        L.csa_index_topk(self.qI, self.w, self.bufs["kidx"], self.k, self.m, fmt=self.fmt,
                         kidx_scale=self.bufs.get("kidx_scale"), idx_out=self.idx, fallback_count=self.fallbacks)
        if ev: ev[3].record()
        L.csa_attend(self.q, self.bufs["entries"], self.idx, m=self.m, win_kv=self.kv_rot, win_roped=True,
                     sink=self.sink, out=self.out)
        if ev: ev[4].record()

    def _cpu_prep(self):
        """Whole-sequence oracle work, done once: compression, the entries'
        bf16 values and the indexer's keys and queries as the kernel sees them."""
        if getattr(self, "_prep", None) is None:
            import oracle as orc
            c = self.c
            t0 = time.time()
            ent, kid = orc.compress(c["kv"][0], c["beta"], self.m, 1, ik=c["ik"][0])
            E = orc.bf16_to_f64(orc.bf16_from_f32(ent))
            qf = orc.bf16_to_f64(c["q_I"][0]).astype(np.float32)
            if self.fmt == "mxfp4":
                kdec = orc.mxfp4_decode(*orc.mxfp4_encode(kid))
                qdec = orc.mxfp4_decode(*orc.mxfp4_encode(qf))
            else:
                kdec = orc.bf16_to_f64(orc.bf16_from_f32(kid)).astype(np.float32)
                qdec = qf
            self._prep = (E, kdec, qdec, time.time() - t0)
        return self._prep

    def row_work(self, rows):
        """Oracle flops of each query row: indexer scores over the visible
        entries, attention over its top-k entries and window."""
        t = np.asarray(rows, dtype=np.int64)
        nv = np.minimum(self.N, (t + 1) // self.m)
        return (2.0 * self.c["H_I"] * 64 * nv
                + 4.0 * self.H * 128 * (np.minimum(self.k, nv) + np.minimum(t + 1, 128)))

    def cpu_baseline(self, sample):
        """The oracle on `sample` query rows drawn uniformly over the sequence,
        extrapolated to all rows by per-row flops, plus the whole-sequence
        compression and encoding (timed whole)."""
        import oracle as orc
        c = self.c
        E, kdec, qdec, t_whole = self._cpu_prep()
        rng = np.random.default_rng(0)
        rows = np.sort(rng.choice(self.n, size=min(sample, self.n), replace=False)).astype(np.int32)
        t1 = time.time()
        idx = orc.index_topk_rows(qdec, c["w_I"][0], kdec, self.m, 0, rows, self.k)
        orc.attend_rows(c["q"][0], 0, E, self.m, rows, "csa", idx=idx, win=c["kv"][0], sink=c["sink"])
        t_rows = time.time() - t1
        frac = self.row_work(rows).sum() / self.row_work(np.arange(self.n)).sum()
        total = t_rows / frac + t_whole
        ext = rows.size < self.n
        return {"value": self.n / total, "extrapolated": ext,
                "sample": "%d of %d query rows%s: oracle top-k + attention (%.2f s)%s, "
                          "plus whole-sequence compression and indexer encoding (%.2f s)"
                          % (rows.size, self.n, " drawn uniformly (seed 0)" if ext else "", t_rows,
                             ", scaled to all rows by per-row flops (indexer scores + attention keys)" if ext
                             else "", t_whole)}


class HcaLayer:
    """Config 2: csa_compress (m' = 128) -> hca_attend."""

    def __init__(self, cfg_id):
        import torch
        import long_context_attention_21_amd as L
        from long_context_attention_21_amd import synth
        self.c = c = synth.config(cfg_id)
        self.L = L
        self.n, self.H, self.m = c["n"], c["H"], c["m"]
        self.q, self.kv = dev_bf16(c["q"]), dev_bf16(c["kv"])
        self.beta, self.sink = dev(c["beta"]), dev(c["sink"])
        N = self.n // self.m
        self.N = N
        self.bufs = {"entries": torch.empty((1, N, 128), dtype=torch.bfloat16, device="cuda")}
        self.out = torch.empty((1, self.n, self.H, 128), dtype=torch.bfloat16, device="cuda")
        self.kernels = ["csa_compress", "csa_rope_rows", "hca_attend"]
        self.kv_rot = torch.empty_like(self.kv)
        self.side = torch.cuda.Stream()
        t = np.arange(self.n, dtype=np.int64)
        keys = int((np.minimum(N, (t + 1) // self.m) + np.minimum(t + 1, 128)).sum())
        self.keys = keys
        # HBM bytes of hca_attend: q in, out back, entries + window rows once.
        # Its arithmetic intensity (about 256 flop/byte) sits below the
        # ridge of 2.5 PFLOP/s / 8 TB/s, so HBM bounds it; MFMA is reported
        # beside.
        self.hca_bytes = 2 * self.n * self.H * 128 * 2 + N * 256 + self.n * 256
        self.work = {
            "csa_compress": ("hbm", self.n * 256 + N * 256),
            "csa_rope_rows": ("hbm", self.n * 512),
            "hca_attend": ("hbm", self.hca_bytes),
        }
        self.work_alt = {"hca_attend": ("bf16", 4.0 * self.H * 128 * keys)}

    def step(self, ev=None):
        """One layer step; without per-kernel events the window rotation runs
        on a side stream beside the compression."""
        L = self.L
        compress = lambda: L.csa_compress(self.kv, self.beta, self.m, 0, out=self.bufs)
        rope = lambda: L.csa_rope_rows(self.kv, out=self.kv_rot)
        if ev is None:
            beside(self.side, rope, compress)
        else:
            ev[0].record()
            compress()
            ev[1].record()
            rope()
            ev[2].record()
        L.hca_attend(self.q, self.bufs["entries"], m=self.m, win_kv=self.kv_rot, win_roped=True, sink=self.sink,
                     out=self.out)
        if ev: ev[3].record()

    def _cpu_prep(self):
        if getattr(self, "_prep", None) is None:
            import oracle as orc
            c = self.c
            t0 = time.time()
            ent, _ = orc.compress(c["kv"][0], c["beta"], self.m, 0)
            self._prep = (orc.bf16_to_f64(orc.bf16_from_f32(ent)), time.time() - t0)
        return self._prep

    def row_work(self, rows):
        t = np.asarray(rows, dtype=np.int64)
        return 4.0 * self.H * 128 * (np.minimum(self.N, (t + 1) // self.m) + np.minimum(t + 1, 128))

    def cpu_baseline(self, sample):
        """The oracle on `sample` query rows (all rows by default), plus the
        whole-sequence compression."""
        import oracle as orc
        c = self.c
        E, t_whole = self._cpu_prep()
        rng = np.random.default_rng(0)
        rows = np.sort(rng.choice(self.n, size=min(sample, self.n), replace=False)).astype(np.int32)
        t1 = time.time()
        orc.attend_rows(c["q"][0], 0, E, self.m, rows, "hca", win=c["kv"][0], sink=c["sink"])
        t_rows = time.time() - t1
        frac = self.row_work(rows).sum() / self.row_work(np.arange(self.n)).sum()
        ext = rows.size < self.n
        return {"value": self.n / (t_rows / frac + t_whole), "extrapolated": ext,
                "sample": "%d of %d query rows%s: oracle attention (%.2f s)%s, plus whole-sequence "
                          "compression (%.2f s)" % (rows.size, self.n, " drawn uniformly (seed 0)" if ext else "",
                                                    t_rows, ", scaled to all rows by per-row flops" if ext else "",
                                                    t_whole)}


def encode_cache(L, entries_bf16, keys_bf16, entry_fmt, out):
    """Store given cache rows in the library's formats: csa_compress with
    m = 1 (one-slot pooling is the identity) and no rotation writes the rows
    as bf16 or FP8 + bf16 entries and MXFP4 indexer keys."""
    import torch
    beta = torch.zeros(1, dtype=torch.float32, device="cuda")
    return L.csa_compress(entries_bf16, beta, 1, 0, ik=keys_bf16, rope_dims=0, entry_fmt=entry_fmt,
                          kidx_fmt="mxfp4", out=out)


class DecodeLayer:
    """Config 4: single-token CSA decode, 64 sequences at t = 1,048,576 over
    262,144 FP8 + bf16 entries (or NVFP4 entries, the V4.1 variant) and MXFP4
    indexer keys each (caches given): csa_index_topk -> csa_attend."""
    entry_fmt = "fp8"

    def __init__(self, cfg_id):
        import torch
        import long_context_attention_21_amd as L
        from long_context_attention_21_amd import synth
        self.L = L
        c = synth.config(cfg_id)
        self.c = c
        B, N, H = c["B"], c["N"], c["H"]
        self.B, self.N, self.H, self.k = B, N, H, c["k"]
        self.n = B  # query tokens per step
        cu = "cuda"
        efmt = self.entry_fmt
        self.codes = torch.empty((B, N, 72 if efmt == "nvfp4" else 64), dtype=torch.uint8, device=cu)
        self.rope = torch.empty((B, N, 64), dtype=torch.bfloat16, device=cu) if efmt == "fp8" else None
        self.scale = torch.empty((B, N), dtype=torch.float32, device=cu)
        self.kc = torch.empty((B, N, 32), dtype=torch.uint8, device=cu)
        self.ks = torch.empty((B, N, 2), dtype=torch.uint8, device=cu)
        self.swa = torch.empty((B, c["n_win"], 128), dtype=torch.bfloat16, device=cu)
        t0 = time.time()
        self.host = []
        for b in range(B):
            ent, ik, swa = c["seq"](b)
            from long_context_attention_21_amd.synth import to_bf16_bits
            e16 = dev_bf16(to_bf16_bits(ent)[None])
            k16 = dev_bf16(to_bf16_bits(ik)[None])
            outs = {"entries": self.codes[b:b + 1], "entry_scale": self.scale[b:b + 1], "kidx": self.kc[b:b + 1],
                    "kidx_scale": self.ks[b:b + 1]}
            if efmt == "fp8":
                outs["entries_rope"] = self.rope[b:b + 1]
            encode_cache(L, e16, k16, efmt, outs)
            self.swa[b] = dev_bf16(swa)
        q, q_I, w_I, sink = c["tail"]()
        self.win8 = self.win8_scale = None
        if efmt == "nvfp4":
            self.make_fp8_window(c)
        log("decode caches generated and stored in %.1f s" % (time.time() - t0))
        self.q, self.qI, self.w, self.sink = dev_bf16(q), dev_bf16(q_I), dev(w_I), dev(sink)
        self.idx = torch.empty((B, 1, self.k), dtype=torch.int32, device=cu)
        self.out = torch.empty((B, 1, H, 128), dtype=torch.bfloat16, device=cu)
        self.fallbacks = torch.zeros(1, dtype=torch.int32, device=cu)  # exact-path work-groups
        self.kernels = ["csa_index_topk", "csa_attend"]
        keys = B * (min(self.k, N) + c["n_win"])
        # bytes: the indexer scans every key (34 B); attention gathers k entries (196 B FP8 + bf16,
        # 76 B NVFP4) + window (256 B bf16, 132 B FP8)
        eb, wb = (76, 132) if efmt == "nvfp4" else (196, 256)
        self.work = {
            "csa_index_topk": ("hbm", B * N * 34),
            "csa_attend": ("hbm", B * (min(self.k, N) * eb + c["n_win"] * wb + 2 * H * 256 + 4 * self.k)),
        }
        self.keys = keys

    def make_fp8_window(self, c):
        """The V4.1 layout's FP8 sliding-window cache: the raw window rows
        appended in order by csa_cache_append into its FP8 ring (an HCA-style
        m = 128 block completes once, into a scratch cache freed after)."""
        import torch
        L, B, W = self.L, self.B, 128
        cu = "cuda"
        ring = torch.zeros((B, 2 * W, 128), dtype=torch.bfloat16, device=cu)
        self.win8 = torch.zeros((B, 2 * W, 128), dtype=torch.uint8, device=cu)
        self.win8_scale = torch.zeros((B, 2 * W), dtype=torch.float32, device=cu)
        beta = torch.zeros(128, dtype=torch.float32, device=cu)
        j0 = c["win_pos0"]
        n_cap = (j0 + c["n_win"]) // 128 + 1
        scratch = {"entries": torch.empty((B, n_cap, 128), dtype=torch.bfloat16, device=cu)}
        for r in range(c["n_win"]):
            L.csa_cache_append(self.swa[:, r].contiguous(), beta, 128, 0, j0 + r, ring, scratch,
                               win8_ring=self.win8, win8_scale=self.win8_scale)
        torch.cuda.synchronize()
        del scratch
        self.win8_pos0 = j0 - (j0 % W)  # ring row s holds position win8_pos0 + s for the window rows

    def step(self, ev=None):
        L, c = self.L, self.c
        if ev: ev[0].record()
        L.csa_index_topk(self.qI, self.w, self.kc, self.k, 4, q_pos0=c["q_pos0"], fmt="mxfp4",
                         kidx_scale=self.ks, idx_out=self.idx, fallback_count=self.fallbacks)
        if ev: ev[1].record()
        if self.win8 is None:
            L.csa_attend(self.q, self.codes, self.idx, q_pos0=c["q_pos0"], m=4, win_kv=self.swa,
                         win_pos0=c["win_pos0"], sink=self.sink, entries_rope=self.rope, entry_scale=self.scale,
                         out=self.out)
        else:  # V4.1 layout: NVFP4 entries, FP8 window ring
            L.csa_attend(self.q, self.codes, self.idx, q_pos0=c["q_pos0"], m=4, win_kv=self.win8,
                         win_pos0=self.win8_pos0, sink=self.sink, entry_scale=self.scale, win_scale=self.win8_scale,
                         out=self.out)
        if ev: ev[2].record()

    def cpu_baseline(self, sample):
        """The oracle on the first `sample` sequences (decoded caches read
        back); every sequence does the same work, so the rate is theirs."""
        import oracle as orc
        c = self.c
        nb = min(sample, self.B)
        t0 = time.time()
        q = self.q.view(torch_int16()).cpu().numpy().view(np.uint16)
        qI = self.qI.view(torch_int16()).cpu().numpy().view(np.uint16)
        w = self.w.cpu().numpy()
        sink = self.sink.cpu().numpy()
        t_rows = 0.0
        for b in range(nb):
            kdec = orc.mxfp4_decode(self.kc[b].cpu().numpy(), self.ks[b].cpu().numpy())
            if self.rope is None:
                E = orc.load_entries_nvfp4(self.codes[b].cpu().numpy(), self.scale[b].cpu().numpy())
            else:
                E = orc.load_entries_fp8(self.codes[b].cpu().numpy(),
                                         self.rope[b].view(torch_int16()).cpu().numpy().view(np.uint16),
                                         self.scale[b].cpu().numpy())
            swa = self.swa[b].view(torch_int16()).cpu().numpy().view(np.uint16)
            wkw = dict(win=swa, win_pos0=c["win_pos0"])
            if self.win8 is not None:
                wkw = dict(win_post=orc.load_window_fp8(self.win8[b].cpu().numpy(), self.win8_scale[b].cpu().numpy()),
                           win_pos0=self.win8_pos0)
            qc, qs = orc.mxfp4_encode(orc.bf16_to_f64(qI[b]).astype(np.float32))
            t1 = time.time()
            rows = np.zeros(1, np.int32)
            idx = orc.index_topk_rows(orc.mxfp4_decode(qc, qs), w[b], kdec, 4, c["q_pos0"], rows, self.k)
            orc.attend_rows(q[b], c["q_pos0"], E, 4, rows, "csa", idx=idx, sink=sink, **wkw)
            t_rows += time.time() - t1
        t_read = time.time() - t0 - t_rows
        return {"value": nb / t_rows, "extrapolated": nb < self.B,
                "sample": "%d of %d sequences: oracle top-k over %d entries + attention for each query (%.2f s)%s; "
                          "reading back and decoding the stored caches (%.1f s) is not charged"
                          % (nb, self.B, self.N, t_rows, ", every sequence the same work" if nb < self.B else "",
                             t_read)}


class PairLayer:
    """Config 5: chunked prefill of one CSA + HCA layer pair, 8192 new tokens
    at P = 1,048,576 over given caches (CSA: 262,144 bf16 entries + MXFP4
    indexer keys, Zipf-skewed; HCA: 8,192 entries) and 128-token state caches.
    CSA: csa_compress (appends 2,048 entries) -> csa_index_topk -> csa_attend;
    HCA: csa_compress (appends 64 entries) -> hca_attend."""

    def __init__(self, cfg_id):
        import torch
        import long_context_attention_21_amd as L
        from long_context_attention_21_amd import synth
        self.L = L
        t0 = time.time()
        c = synth.config(cfg_id)
        self.c = c
        cs, hs = c["csa"], c["hca"]
        n, P, H, k = c["n"], c["P"], c["H"], c["k"]
        self.n, self.P, self.H, self.k = n, P, H, k
        Nc0, Nh0 = c["N_csa_prior"], c["N_hca_prior"]
        self.Nc, self.Nh = Nc0 + n // 4, Nh0 + n // 128
        self.Nc0, self.Nh0 = Nc0, Nh0
        cu = "cuda"
        # CSA caches: prior rows stored by the library's encoder, room for the chunk's entries
        self.c_ent = torch.empty((1, self.Nc, 128), dtype=torch.bfloat16, device=cu)
        self.c_kc = torch.empty((1, self.Nc, 32), dtype=torch.uint8, device=cu)
        self.c_ks = torch.empty((1, self.Nc, 2), dtype=torch.uint8, device=cu)
        encode_cache(L, dev_bf16(cs["entries_prior"][None]),
                     dev_bf16(synth.to_bf16_bits(cs["kI_prior_f32"])[None]), "bf16",
                     {"entries": self.c_ent[:, :Nc0], "kidx": self.c_kc[:, :Nc0], "kidx_scale": self.c_ks[:, :Nc0]})
        # window sources: state (positions P-128 .. P-1) followed by the chunk
        self.c_win = dev_bf16(np.concatenate([cs["state_kv"], cs["kv_new"]])[None])
        self.c_ik = dev_bf16(np.concatenate([cs["state_ik"], cs["ik_new"]])[None])
        self.c_q, self.c_qI, self.c_w = dev_bf16(cs["q"][None]), dev_bf16(cs["q_I"][None]), dev(cs["w_I"][None])
        self.c_beta, self.c_sink = dev(cs["beta"]), dev(cs["sink"])
        self.h_ent = torch.empty((1, self.Nh, 128), dtype=torch.bfloat16, device=cu)
        self.h_ent[:, :Nh0] = dev_bf16(hs["entries_prior"][None])
        self.h_win = dev_bf16(np.concatenate([hs["state_kv"], hs["kv_new"]])[None])
        self.h_q, self.h_beta, self.h_sink = dev_bf16(hs["q"][None]), dev(hs["beta"]), dev(hs["sink"])
        self.idx = torch.empty((1, n, k), dtype=torch.int32, device=cu)
        self.fallbacks = torch.zeros(1, dtype=torch.int32, device=cu)  # exact-path work-groups
        self.c_out = torch.empty((1, n, H, 128), dtype=torch.bfloat16, device=cu)
        self.h_out = torch.empty((1, n, H, 128), dtype=torch.bfloat16, device=cu)
        self.calls = 0
        log("pair inputs generated in %.1f s" % (time.time() - t0))
        self.kernels = ["csa_compress", "csa_rope_rows", "csa_index_topk", "csa_attend", "hca_compress",
                        "hca_rope_rows", "hca_attend"]
        self.c_rot = torch.empty_like(self.c_win)
        self.h_rot = torch.empty_like(self.h_win)
        t = P + np.arange(n, dtype=np.int64)
        nv = np.minimum(self.Nc, (t + 1) // 4)
        pairs = int(nv.sum())
        keys_c = int((np.minimum(k, nv) + 128).sum())
        keys_h = int((np.minimum(self.Nh, (t + 1) // 128) + 128).sum())
        self.work = {
            "csa_compress": ("hbm", n * (256 + 128) + (n // 4) * (256 + 34)),
            "csa_rope_rows": ("hbm", (n + 128) * 512),
            "csa_index_topk": ("fp4", 2.0 * 8 * 64 * pairs),
            "csa_attend": ("bf16", 4.0 * H * 128 * keys_c),
            "hca_compress": ("hbm", n * 256 + (n // 128) * 256),
            "hca_rope_rows": ("hbm", (n + 128) * 512),
            "hca_attend": ("bf16", 4.0 * H * 128 * keys_h),
        }

    # csa_index_attend's token chunks for the CSA layer.  1 (the calls in
    # turn): a chunk of this layer's rows, which see up to 262144 entries
    # each, has too few long indexer work-groups to fill the GPU, so chunks
    # add their tails (measured 6.0-6.2 ms/step in turn, 6.2 / 7.9 / 9.0 ms
    # with 2 / 4 / 8 chunks)
    chunks = 1

    def step(self, ev=None, serial=False):
        """One step of the pair.  With per-kernel events (or serial) every
        call runs in turn; otherwise the CSA layer's indexer and attention
        run as csa_index_attend over self.chunks token chunks."""
        L, P, n = self.L, self.P, self.n
        self.calls += 1
        if ev: ev[0].record()
        L.csa_compress(self.c_win[:, 128:], self.c_beta, 4, 1, pos0=P, ik=self.c_ik[:, 4:],
                       prev_kv=self.c_win[:, 124:128], prev_ik=self.c_ik[:, :4], kidx_fmt="mxfp4",
                       out={"entries": self.c_ent[:, self.Nc0:], "kidx": self.c_kc[:, self.Nc0:],
                            "kidx_scale": self.c_ks[:, self.Nc0:]})
        if ev: ev[1].record()
        L.csa_rope_rows(self.c_win, pos0=P - 128, out=self.c_rot)
        if ev: ev[2].record()
        if ev is None and not serial and self.chunks > 1:
            L.csa_index_attend(self.c_qI, self.c_w, self.c_kc, self.k, 4, self.c_q, self.c_ent, q_pos0=P,
                               fmt="mxfp4", kidx_scale=self.c_ks, idx_out=self.idx, fallback_count=self.fallbacks,
                               win_kv=self.c_rot, win_pos0=P - 128, win_roped=True, sink=self.c_sink,
                               out=self.c_out, n_chunks=self.chunks)
        else:
            L.csa_index_topk(self.c_qI, self.c_w, self.c_kc, self.k, 4, q_pos0=P, fmt="mxfp4",
                             kidx_scale=self.c_ks, idx_out=self.idx, fallback_count=self.fallbacks)
            if ev: ev[3].record()
            L.csa_attend(self.c_q, self.c_ent, self.idx, q_pos0=P, m=4, win_kv=self.c_rot, win_pos0=P - 128,
                         win_roped=True, sink=self.c_sink, out=self.c_out)
        if ev: ev[4].record()
        L.csa_compress(self.h_win[:, 128:], self.h_beta, 128, 0, pos0=P, out={"entries": self.h_ent[:, self.Nh0:]})
        if ev: ev[5].record()
        L.csa_rope_rows(self.h_win, pos0=P - 128, out=self.h_rot)
        if ev: ev[6].record()
        L.hca_attend(self.h_q, self.h_ent, q_pos0=P, m=128, win_kv=self.h_rot, win_pos0=P - 128,
                     win_roped=True, sink=self.h_sink, out=self.h_out)
        if ev: ev[7].record()

    def _cpu_prep(self):
        """The chunk's compression (both layers) and the caches as the
        kernels see them, done once."""
        if getattr(self, "_prep", None) is None:
            import oracle as orc
            cs, hs = self.c["csa"], self.c["hca"]
            t0 = time.time()
            ent_new, kid_new = orc.compress(cs["kv_new"], cs["beta"], 4, 1, pos0=self.P, ik=cs["ik_new"],
                                            prev_kv=cs["state_kv"][124:], prev_ik=cs["state_ik"])
            hent_new, _ = orc.compress(hs["kv_new"], hs["beta"], 128, 0, pos0=self.P)
            t_comp = time.time() - t0
            E = np.concatenate([orc.bf16_to_f64(cs["entries_prior"]),
                                orc.bf16_to_f64(orc.bf16_from_f32(ent_new))])
            kq, ks = orc.mxfp4_encode(orc.bf16_to_f64(orc.bf16_from_f32(cs["kI_prior_f32"])).astype(np.float32))
            kn, ksn = orc.mxfp4_encode(kid_new)
            kdec = np.concatenate([orc.mxfp4_decode(kq, ks), orc.mxfp4_decode(kn, ksn)])
            qdec = orc.mxfp4_decode(*orc.mxfp4_encode(orc.bf16_to_f64(cs["q_I"]).astype(np.float32)))
            HE = np.concatenate([orc.bf16_to_f64(hs["entries_prior"]),
                                 orc.bf16_to_f64(orc.bf16_from_f32(hent_new))])
            self._prep = (E, kdec, qdec, HE, t_comp, time.time() - t0 - t_comp)
        return self._prep

    def row_work(self, rows):
        t = self.P + np.asarray(rows, dtype=np.int64)
        nv = np.minimum(self.Nc, (t + 1) // 4)
        return (2.0 * 8 * 64 * nv + 4.0 * self.H * 128 * (np.minimum(self.k, nv) + 128)
                + 4.0 * self.H * 128 * (np.minimum(self.Nh, (t + 1) // 128) + 128))

    def cpu_baseline(self, sample):
        """The oracle on `sample` query rows of the chunk (both layers),
        extrapolated to the chunk by per-row flops, plus the chunk's
        compression (timed whole); decoding the prior caches is not charged."""
        import oracle as orc
        cs, hs = self.c["csa"], self.c["hca"]
        E, kdec, qdec, HE, t_comp, t_dec = self._cpu_prep()
        rng = np.random.default_rng(0)
        rows = np.sort(rng.choice(self.n, size=min(sample, self.n), replace=False)).astype(np.int32)
        win_c = np.concatenate([cs["state_kv"], cs["kv_new"]])
        win_h = np.concatenate([hs["state_kv"], hs["kv_new"]])
        t1 = time.time()
        idx = orc.index_topk_rows(qdec, cs["w_I"], kdec, 4, self.P, rows, self.k)
        orc.attend_rows(cs["q"], self.P, E, 4, rows, "csa", idx=idx, win=win_c, win_pos0=self.P - 128,
                        sink=cs["sink"])
        orc.attend_rows(hs["q"], self.P, HE, 128, rows, "hca", win=win_h, win_pos0=self.P - 128, sink=hs["sink"])
        t_rows = time.time() - t1
        frac = self.row_work(rows).sum() / self.row_work(np.arange(self.n)).sum()
        ext = rows.size < self.n
        return {"value": self.n / (t_rows / frac + t_comp), "extrapolated": ext,
                "sample": "%d of %d query rows of the chunk drawn uniformly (seed 0): oracle CSA top-k + CSA "
                          "attention + HCA attention (%.2f s)%s, plus the chunk's compression (%.2f s); decoding "
                          "the prior caches (%.1f s) is not charged"
                          % (rows.size, self.n, t_rows, ", scaled to the chunk by per-row flops" if ext else "",
                             t_comp, t_dec)}


def torch_int16():
    import torch
    return torch.int16


WORKLOAD = {
    1: "CSA layer forward, batch 1, 1024 tokens, 8 heads x 128, m=4 overlapped, bf16 indexer 4x64, top-k 64, SWA 128, sink",
    4: "CSA decode, 64 sequences x 1 token at t=1048576, 262144 FP8+bf16 entries + MXFP4 indexer keys each, top-k 2048, SWA 128, sink",
    5: "CSA+HCA layer pair, chunked prefill of 8192 tokens at P=1048576 (CSA 262144 prior entries, Zipf-skewed indexer keys; HCA 8192 prior entries), 64 heads, top-k 2048, SWA 128, sink",
    2: "HCA layer forward, batch 1, 32768 tokens, 64 heads x 128, m'=128 (256 entries), SWA 128, sink",
    3: "CSA prefill, batch 1, 131072 tokens, 64 heads x 128, m=4 overlapped (32768 entries), MXFP4 indexer 8x64, top-k 2048, SWA 128, sink",
}


DTYPE = {1: "bf16", 2: "bf16", 3: "bf16 (attention MFMA) + mxfp4 (indexer MFMA)",
         4: "fp8 e4m3 + bf16 entries, bf16 MFMA (attention) + mxfp4 (indexer MFMA)",
         5: "bf16 (attention MFMA) + mxfp4 (indexer MFMA)"}
CPU_SAMPLE = {1: 1024, 2: 32768, 3: 8192, 4: 16, 5: 1024}  # query rows (config 4: sequences)
CPU_SAMPLE_1T = {1: 128, 2: 512, 3: 256, 4: 2, 5: 32}  # the same at one thread
# the two HBM-bound workloads timed beside the default one, under these names
EXTRA = (("hca_prefill_32k", 2), ("csa_decode_64x1m", 4))


def cpu_leg(wl, cfg_id, sample):
    """The oracle on a bounded sample of the workload: all host cores, then
    one thread on a smaller sample."""
    import oracle
    oracle.build()
    log("cpu baseline: oracle on %d sampled %s" % (sample, "sequences" if cfg_id == 4 else "query rows"))
    r = wl.cpu_baseline(sample)
    cpu = {"value": round(r["value"], 2), "unit": "query-tokens/s", "cores": _cores(), "kind": "oracle",
           "extrapolated": r["extrapolated"], "sample": r["sample"]}
    prev = oracle.set_threads(1)
    try:
        r1 = wl.cpu_baseline(min(sample, CPU_SAMPLE_1T[cfg_id]))
    finally:
        oracle.set_threads(prev)
    cpu["one_thread"] = {"value": round(r1["value"], 2), "cores": 1, "extrapolated": r1["extrapolated"],
                         "sample": r1["sample"]}
    return cpu


# wall time of warmup at least, per workload: the HCA and decode steps last
# 0.2-0.6 ms, and a few of them do not bring the GPU clock up
MIN_WARM_S = {2: 0.5, 4: 0.5}


def measure(cfg_id, args, cpu_sample=None):
    """Warm up, time args.steps steps of workload `cfg_id` (per-kernel HIP
    events on the launch stream), then the oracle baseline.  After the
    args.warmup steps, short-step workloads keep warming up until
    MIN_WARM_S of wall time has passed;
    the count actually run is reported as `warmup` (MIN_WARM_S)."""
    import torch
    min_warm_s = MIN_WARM_S.get(cfg_id, 0.0)
    wl = {1: CsaLayer, 2: HcaLayer, 3: CsaLayer, 4: DecodeLayer, 5: PairLayer}[cfg_id](cfg_id)
    nk = len(wl.kernels)
    log("config %d: warmup %d steps" % (cfg_id, args.warmup))
    tw = time.perf_counter()
    warm = 0
    while warm < args.warmup or time.perf_counter() - tw < min_warm_s:
        wl.step()
        warm += 1
        if warm >= args.warmup:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(args.steps)]
    # The steps are timed as a whole with nothing but the launches in the
    # timed region; the per-kernel figures come from a second pass of the
    # same number of steps with a HIP event between the calls.  A pipelined
    # step (csa_index_attend) overlaps the indexer and the attention, so its
    # second pass runs the calls in turn.
    piped = getattr(wl, "chunks", 1) > 1
    log("config %d: timing %d steps" % (cfg_id, args.steps))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        wl.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log("config %d: per-kernel pass, %d steps%s" % (cfg_id, args.steps, " with the calls in turn" if piped else ""))
    if piped:
        wl.step(serial=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s in range(args.steps):
        wl.step(evs[s])
    torch.cuda.synchronize()
    pass_ms = (time.perf_counter() - t1) * 1e3 / args.steps
    per_k = np.zeros(nk)
    for s in range(args.steps):
        for i in range(nk):
            per_k[i] += evs[s][i].elapsed_time(evs[s][i + 1])
    per_k /= args.steps  # ms per launch
    ms_step = wall * 1e3 / args.steps

    kernels = {}
    for i, name in enumerate(wl.kernels):
        kind, amount = wl.work[name]
        sec = per_k[i] / 1e3
        if kind == "hbm":
            ach, peak, unit = amount / sec / 1e9, PEAK["hbm"], "GB/s"
        else:
            ach, peak, unit = amount / sec / 1e12, PEAK[kind], "TFLOP/s"
        kernels[name] = {"ms": round(per_k[i], 4), "bound": "hbm" if kind == "hbm" else "mfma",
                         "dtype": kind, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                         "frac": round(ach / peak, 4), "work": amount,
                         "traffic": traffic_bytes(name, cfg_id)}
        alt = getattr(wl, "work_alt", {}).get(name)
        if alt:  # the other roof of the same launch
            akind, aamount = alt
            aach = aamount / sec / 1e12
            kernels[name]["also"] = {"bound": "mfma", "dtype": akind, "achieved": round(aach, 2),
                                     "peak": PEAK[akind], "unit": "TFLOP/s", "frac": round(aach / PEAK[akind], 4),
                                     "work": aamount}
    dom = wl.kernels[int(np.argmax(per_k))]
    dk = kernels[dom]
    roofline = {"kernel": dom, "bound": dk["bound"], "achieved": dk["achieved"], "peak": dk["peak"],
                "unit": dk["unit"], "frac": dk["frac"], "traffic": traffic_bytes(dom, cfg_id)}
    cpu = None
    if not args.no_cpu:
        cpu = cpu_leg(wl, cfg_id, cpu_sample or CPU_SAMPLE[cfg_id])

    wname, dname = WORKLOAD[cfg_id], DTYPE[cfg_id]
    if cfg_id == 4 and DecodeLayer.entry_fmt == "nvfp4":
        wname = wname.replace("262144 FP8+bf16 entries", "262144 NVFP4 entries + an FP8 window cache "
                                                         "(post-RoPE, the V4.1 variant)")
        dname = dname.replace("fp8 e4m3 + bf16 entries", "nvfp4 entries")
    cfg = {"workload": wname, "global_batch": getattr(wl, "B", 1), "seq_len": wl.n,
           "heads": wl.H, "head_dim": 128}
    res = {"value": round(wl.n / (ms_step / 1e3), 1), "unit": "query-tokens/s", "steps": args.steps,
           "warmup": warm, "ms_per_step": round(ms_step, 4), "dtype": dname, "config": cfg,
           "roofline": roofline, "kernels": kernels, "cpu_baseline": cpu}
    if piped:
        res["schedule"] = {
            "step": "csa_compress with csa_rope_rows beside it on a side stream, then csa_index_attend: %d token "
                    "chunks, the indexer of chunk c + 1 on a second stream beside the attention of chunk c"
                    % wl.chunks,
            "kernels_and_roofline": "per-launch durations from a second pass of %d steps with the four calls in "
                                    "turn on one stream, HIP events between them" % args.steps,
            "serial_ms_per_step": round(pass_ms, 4)}
    else:
        res["schedule"] = {
            "kernels_and_roofline": "per-launch durations from a second pass of %d steps with HIP events between "
                                    "the calls" % args.steps,
            "events_ms_per_step": round(pass_ms, 4)}
    if hasattr(wl, "fallbacks"):  # top-k work-groups that took the exact streaming path, per call
        ncalls = getattr(wl, "calls", warm + 2 * args.steps)  # warmup, the timed steps and the per-kernel pass
        res["topk_fallbacks_per_call"] = round(int(wl.fallbacks.item()) / ncalls, 2)
    del wl
    torch.cuda.empty_cache()
    return res


def _grid(row):
    grid = "x".join(row[c] for c in ("Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z") if c in row)
    return grid or row.get("Grid_Size", "?")


def trace_summary(path):
    """Dispatches, total and average duration (us) per (kernel, grid size)
    of a rocprofv3 --kernel-trace CSV (or, for a --pmc counter_collection
    CSV, each counter's mean value per dispatch): the pipelined step's
    chunked launches and the per-kernel pass's whole-layer launches of one
    kernel have different grids."""
    import csv
    with open(path, newline="") as f:
        rows = list(csv.DictReader(f))
    if rows and "Counter_Name" in rows[0]:
        per = {}  # (kernel, grid) -> counter -> dispatch -> value
        for row in rows:
            d = per.setdefault((row["Kernel_Name"], _grid(row)), {}).setdefault(row["Counter_Name"], {})
            d[row["Dispatch_Id"]] = d.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
        print("%-66s %14s %6s %-28s %16s" % ("kernel", "grid", "n", "counter", "mean_per_dispatch"))
        for (name, grid), cs in sorted(per.items()):
            for cname, disp in sorted(cs.items()):
                print("%-66s %14s %6d %-28s %16.6g" % (name[:66], grid, len(disp), cname,
                                                       sum(disp.values()) / len(disp)))
        return
    groups = {}
    if True:
        for row in rows:
            grid = _grid(row)
            dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
            g = groups.setdefault((row["Kernel_Name"], grid), [0, 0.0])
            g[0] += 1
            g[1] += dur
    total = sum(v[1] for v in groups.values())
    print("%-66s %14s %6s %12s %11s %6s" % ("kernel", "grid", "calls", "total_us", "average_us", "pct"))
    for (name, grid), (cnt, us) in sorted(groups.items(), key=lambda kv: -kv[1][1]):
        print("%-66s %14s %6d %12.1f %11.1f %6.2f" % (name[:66], grid, cnt, us, us / cnt, 100 * us / total))


def main():
    args = parse()
    if args.print_sha:
        print(json.dumps({k: source_sha(k) for k in KERNEL_SOURCE}))
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "no GPU"
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe()
        return
    if args.append_probe:
        append_probe(no_cpu=args.no_cpu)
        return
    if args.proj_probe:
        proj_probe(no_cpu=args.no_cpu)
        return
    if args.entry_fmt != "fp8":
        if args.config != 4:
            sys.exit("--entry-fmt applies to config 4 only")
        DecodeLayer.entry_fmt = args.entry_fmt
    if args.chunks is not None:
        CsaLayer.chunks = PairLayer.chunks = max(1, args.chunks)
    cfg_id = args.config or 3
    res = measure(cfg_id, args, args.cpu_sample)
    line = {
        "metric": METRIC, "value": res["value"], "unit": res["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": res["warmup"], "ms_per_step": res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": res["dtype"], "data": "synthetic (seeded, numpy default_rng)", "config": res["config"],
        "roofline": res["roofline"], "kernels": res["kernels"], "cpu_baseline": res["cpu_baseline"],
    }
    for key in ("schedule", "topk_fallbacks_per_call"):
        if key in res:
            line[key] = res[key]
    if args.config is None and not args.no_extra:
        line["workloads"] = {name: measure(c, args) for name, c in EXTRA}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
