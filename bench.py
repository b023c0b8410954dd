"""Benchmark of the hybrid compressed attention forward on one MI355X.

Default workload (the 128K-context configuration): one CSA layer prefill,
batch 1, 131072 query tokens, 64 heads of dim 128 with RoPE on the last 64
dims, m = 4 overlapped compression (32768 entries), MXFP4 Lightning Indexer
(8 heads x 64, q quantised in-kernel), top-k 2048, 128-token window, per-head
sink.  One step = csa_compress -> csa_index_topk -> csa_attend over the whole
sequence, inputs resident in HBM.  --config 2 times the HCA layer (32768
tokens, m' = 128), --config 1 the small CSA layer.

Prints one JSON line: throughput (query tokens/s), the roofline of the
dominant kernel (per-kernel durations from HIP events recorded on the launch
stream over the timed region), per-kernel figures, and the CPU oracle timed
on a bounded sample of the same workload (rank 0, N = 1 only).
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
# (scaled by the plain-copy calibration of --copy-probe), keyed by the
# sha256 of the kernel source they were taken on: a changed kernel reports
# null until it is measured again.
TRAFFIC = {  # profiles/csa_prefill_128k_hbm_counters.txt
    ("csa_attend", 3): {"sha256": "9eea36c3279a74f73dae90780ffc27f42e859a4a1dc7597a592f457362a2c3c5",
                        "bytes": 1.852e10},
    ("csa_index_topk", 3): {"sha256": "ea442c78d7fa3476a387827a409882b532a752cc74ff43be7668878dfc8062eb",
                            "bytes": 1.219e9},
    ("csa_compress", 3): {"sha256": "82c3e1fea99ff0128101cd4a89cfefe6bb708f379c3a3e689974d4dc357c12da",
                          "bytes": 7.279e7},
}
KERNEL_SOURCE = {"csa_compress": "compress.hip", "csa_index_topk": "index_topk.hip",
                 "csa_attend": "attend.hip", "hca_attend": "attend.hip"}


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
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3])
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="query rows of the oracle sample (default per config)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only copy 1 GiB device-to-device 3 times (HBM counter calibration)")
    ap.add_argument("--print-sha", action="store_true", help="print the kernel source hashes and exit")
    return ap.parse_args()


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


# ---------------------------------------------------------------- workloads --

def dev_bf16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


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
        self.kernels = ["csa_compress", "csa_index_topk", "csa_attend"]
        # algorithmic work (measurement)
        t = np.arange(n, dtype=np.int64)
        nv = np.minimum(N, (t + 1) // self.m)
        pairs = int(nv.sum())
        keys = int((np.minimum(self.k, nv) + np.minimum(t + 1, 128)).sum())
        kbytes = 34 if self.fmt == "mxfp4" else 128
        self.work = {
            "csa_compress": ("hbm", n * (256 + 128) + N * (256 + kbytes)),
            "csa_index_topk": ("fp4" if self.fmt == "mxfp4" else "bf16", 2.0 * 8 * 64 * pairs
                               if self.fmt == "mxfp4" else 2.0 * c["H_I"] * 64 * pairs),
            "csa_attend": ("bf16", 4.0 * self.H * 128 * keys),
        }
        self.pairs, self.keys = pairs, keys

    def step(self, ev=None):
        L = self.L
        if ev: ev[0].record()
        L.csa_compress(self.kv, self.beta, self.m, 1, ik=self.ik, kidx_fmt=self.fmt, out=self.bufs)
        if ev: ev[1].record()
        L.csa_index_topk(self.qI, self.w, self.bufs["kidx"], self.k, self.m, fmt=self.fmt,
                         kidx_scale=self.bufs.get("kidx_scale"), idx_out=self.idx)
        if ev: ev[2].record()
        L.csa_attend(self.q, self.bufs["entries"], self.idx, m=self.m, win_kv=self.kv,
                     sink=self.sink, out=self.out)
        if ev: ev[3].record()

    def cpu_baseline(self, sample):
        """The oracle on `sample` query rows spread over the sequence (plus the
        compression of the whole sequence, charged pro rata)."""
        import oracle as orc
        c = self.c
        rng = np.random.default_rng(0)
        rows = np.sort(rng.choice(self.n, size=min(sample, self.n), replace=False)).astype(np.int32)
        t0 = time.time()
        ent, kid = orc.compress(c["kv"][0], c["beta"], self.m, 1, ik=c["ik"][0])
        t_comp = time.time() - t0
        E = orc.bf16_to_f64(orc.bf16_from_f32(ent))
        qf = orc.bf16_to_f64(c["q_I"][0]).astype(np.float32)
        if self.fmt == "mxfp4":
            kc, ks = orc.mxfp4_encode(kid)
            kdec = orc.mxfp4_decode(kc, ks)
            qc, qs = orc.mxfp4_encode(qf)
            qdec = orc.mxfp4_decode(qc, qs)
        else:
            kdec = orc.bf16_to_f64(orc.bf16_from_f32(kid)).astype(np.float32)
            qdec = qf
        t_prep = time.time() - t0 - t_comp
        t1 = time.time()
        idx = orc.index_topk_rows(qdec, c["w_I"][0], kdec, self.m, 0, rows, self.k)
        _ = orc.attend_rows(c["q"][0], 0, E, self.m, rows, "csa", idx=idx, win=c["kv"][0],
                            sink=c["sink"])
        t_rows = time.time() - t1
        total = t_rows + (t_comp + t_prep) * rows.size / self.n
        return rows.size / total, rows.size, t_comp + t_prep, t_rows


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
        self.kernels = ["csa_compress", "hca_attend"]
        t = np.arange(self.n, dtype=np.int64)
        keys = int((np.minimum(N, (t + 1) // self.m) + np.minimum(t + 1, 128)).sum())
        self.keys = keys
        self.work = {
            "csa_compress": ("hbm", self.n * 256 + N * 256),
            "hca_attend": ("bf16", 4.0 * self.H * 128 * keys),
        }
        # HBM bytes of hca_attend: q in, out back, entries + raw rows once
        self.hca_bytes = 2 * self.n * self.H * 128 * 2 + N * 256 + self.n * 256

    def step(self, ev=None):
        L = self.L
        if ev: ev[0].record()
        L.csa_compress(self.kv, self.beta, self.m, 0, out=self.bufs)
        if ev: ev[1].record()
        L.hca_attend(self.q, self.bufs["entries"], m=self.m, win_kv=self.kv, sink=self.sink,
                     out=self.out)
        if ev: ev[2].record()

    def cpu_baseline(self, sample):
        import oracle as orc
        c = self.c
        rng = np.random.default_rng(0)
        rows = np.sort(rng.choice(self.n, size=min(sample, self.n), replace=False)).astype(np.int32)
        t0 = time.time()
        ent, _ = orc.compress(c["kv"][0], c["beta"], self.m, 0)
        t_comp = time.time() - t0
        E = orc.bf16_to_f64(orc.bf16_from_f32(ent))
        t1 = time.time()
        orc.attend_rows(c["q"][0], 0, E, self.m, rows, "hca", win=c["kv"][0], sink=c["sink"])
        t_rows = time.time() - t1
        total = t_rows + t_comp * rows.size / self.n
        return rows.size / total, rows.size, t_comp, t_rows


WORKLOAD = {
    1: "CSA layer forward, batch 1, 1024 tokens, 8 heads x 128, m=4 overlapped, bf16 indexer 4x64, top-k 64, SWA 128, sink",
    2: "HCA layer forward, batch 1, 32768 tokens, 64 heads x 128, m'=128 (256 entries), SWA 128, sink",
    3: "CSA prefill, batch 1, 131072 tokens, 64 heads x 128, m=4 overlapped (32768 entries), MXFP4 indexer 8x64, top-k 2048, SWA 128, sink",
}


def main():
    args = parse()
    if args.print_sha:
        print(json.dumps({k: source_sha(k) for k in KERNEL_SOURCE}))
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
    wl = CsaLayer(args.config) if args.config in (1, 3) else HcaLayer(args.config)
    nk = len(wl.kernels)
    log("warmup %d steps" % args.warmup)
    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(args.steps)]
    log("timing %d steps" % args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        wl.step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_k = np.zeros(nk)
    for s in range(args.steps):
        for i in range(nk):
            per_k[i] += evs[s][i].elapsed_time(evs[s][i + 1])
    per_k /= args.steps  # ms per launch
    ms_step = wall * 1e3 / args.steps
    value = wl.n / (ms_step / 1e3)

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
                         "traffic": traffic_bytes(name, args.config)}
    dom = wl.kernels[int(np.argmax(per_k))]
    dk = kernels[dom]
    roofline = {"kernel": dom, "bound": dk["bound"], "achieved": dk["achieved"], "peak": dk["peak"],
                "unit": dk["unit"], "frac": dk["frac"], "traffic": traffic_bytes(dom, args.config)}

    cpu = None
    if not args.no_cpu:
        sample = args.cpu_sample or {1: 1024, 2: 32768, 3: 8192}[args.config]
        log("cpu baseline: oracle on %d sampled query rows" % sample)
        import oracle
        oracle.build()
        v, rows, t_comp, t_rows = wl.cpu_baseline(sample)
        cores = len(os.sched_getaffinity(0))
        omp = os.environ.get("OMP_NUM_THREADS")
        if omp:
            cores = min(cores, int(omp))
        cpu = {"value": round(v, 2), "unit": "query-tokens/s", "cores": cores, "kind": "oracle",
               "sample": "%d query rows drawn uniformly over the sequence (seed 0): oracle top-k + "
                         "attention for those rows (%.1f s) plus whole-sequence compression "
                         "(%.1f s) charged pro rata" % (rows, t_rows, t_comp)}

    cfg = {"workload": WORKLOAD[args.config], "global_batch": 1, "seq_len": wl.n,
           "heads": wl.H, "head_dim": 128}
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 (attention MFMA) + mxfp4 (indexer MFMA)" if args.config == 3 else "bf16",
        "data": "synthetic (seeded, numpy default_rng)", "config": cfg,
        "roofline": roofline, "kernels": kernels, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
