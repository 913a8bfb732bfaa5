#!/usr/bin/env python3
"""Benchmark of the IndexPool sparse-attention decode step on one MI355X.

Headline: sparse-attention decode steps/s at 1M-token context (top 512 groups =
2048 tokens) and the achieved HBM bandwidth, on the 8 x 1,048,576-token decode
workload.  One step = isa_indexer_topk (score every pooled group of every
sequence and select the top 512) + isa_sparse_mla_decode (64-head NoPE MLA over
the selected latent rows) for the whole batch; the pooled int8 key cache is
built beforehand by isa_indexpool, as a serving engine would keep it.

Inputs are seeded synthetic tensors resident in HBM before the timed region.
Four copies of the pooled cache (1 GiB) and 16 query sets rotate across steps
so that neither the keys nor the gathered latent rows are served from the
256 MB Infinity Cache.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

METRIC = "sparse-attn decode steps/s at 1M ctx (top-2048) + achieved HBM GB/s"
HBM_PEAK_GBPS = 8000.0
INT8_PEAK_TOPS = 5000.0
N_POOL_COPIES = 4
N_QSETS = 16
KERNEL_SOURCES = {
    "k_indexer_decode": ["indexer_decode.hip", "select_device.hpp", "isa_common.hpp", "isa_launch.hpp"],
}


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(ROOT, "long_context_sparse_indexpool_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("source_hash") != source_hash(kernel):
        return None
    return d.get("hbm_bytes_per_launch")


class Decode:
    """Device state of one decode workload with rotation sets."""

    def __init__(self, wl, n_copies, n_qsets, keep_host=False):
        import numpy as np
        import torch

        import harness as H
        import long_context_sparse_indexpool_amd as m
        from synth.configs import LAT_DIM

        self.wl, self.m, self.torch = wl, m, torch
        B = wl.batch
        t0 = time.time()
        db = H.make_batch(wl, with_keys=True, with_latent=True, keep_host=keep_host)
        log(f"{wl.name}: inputs generated and uploaded in {time.time() - t0:.1f}s")
        H.run_pool(db)
        self.db = db
        self.pooled = [db.pooled] + [db.pooled.clone() for _ in range(n_copies - 1)]
        del db.keys
        db.keys = None
        torch.cuda.empty_cache()
        self.q = [torch.from_numpy(wl.q_idx(B * i, B)).cuda() for i in range(n_qsets)]
        self.hw = [torch.from_numpy(wl.head_w(B * i, B)).cuda() for i in range(n_qsets)]
        self.qa = [torch.from_numpy(wl.q_attn(B * i, B).view(np.int16)).cuda() for i in range(n_qsets)]
        self.k = 512
        self.idx = torch.zeros((B, self.k), dtype=torch.int32, device="cuda")
        self.cnt = torch.zeros(B, dtype=torch.int32, device="cuda")
        self.out = torch.zeros((B, 64, LAT_DIM), dtype=torch.float32, device="cuda")
        self.lse = torch.zeros((B, 64), dtype=torch.float32, device="cuda")
        self.ws_topk = m.alloc_workspace(m.workspace_size(m.ISA_OP_INDEXER_TOPK, db.seqs))
        self.ws_att = m.alloc_workspace(m.workspace_size(m.ISA_OP_SPARSE_MLA, db.seqs, B))
        self.i = 0
        G = [wl.groups(b) for b in range(B)]
        sel_tok = [min(L, 4 * self.k) for L in wl.lens]  # tokens gathered (dense rows: all of them)
        # algorithmic bytes of one step
        self.bytes_topk = sum(128 * g for g in G if g > self.k) + B * (32 * 128 + 32) + B * (self.k * 4 + 4)
        self.bytes_att = sum(1024 * t for t in sel_tok) + B * (64 * 512 * 2 + 64 * 512 * 4 + 64 * 4) + \
            B * (self.k * 4 + 4)
        self.bytes_step = self.bytes_topk + self.bytes_att

    def topk(self, j):
        m = self.m
        B = self.wl.batch
        m.isa_indexer_topk(self.q[j % len(self.q)], self.hw[j % len(self.hw)], self.pooled[j % len(self.pooled)],
                           self.db.seqs, None, B, 0, self.k, self.idx, self.cnt, None, self.ws_topk)

    def attention(self, j):
        from synth.configs import SM_SCALE
        m = self.m
        B = self.wl.batch
        m.isa_sparse_mla_decode(self.qa[j % len(self.qa)], self.db.latent, self.db.seqs, None, None, B, self.idx,
                                self.cnt, self.k, SM_SCALE, self.out, self.lse, self.ws_att)

    def step(self):
        self.topk(self.i)
        self.attention(self.i)
        self.i += 1

    def time_steps(self, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    def time_kernels(self, reps):
        """Average durations of the indexer launch and of the attention launches,
        with HIP events on the stream the library launches on."""
        torch = self.torch
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * reps)]
        for r in range(reps):
            ev[3 * r].record()
            self.topk(self.i)
            ev[3 * r + 1].record()
            self.attention(self.i)
            ev[3 * r + 2].record()
            self.i += 1
        torch.cuda.synchronize()
        t_topk = sum(ev[3 * r].elapsed_time(ev[3 * r + 1]) for r in range(reps)) / reps
        t_att = sum(ev[3 * r + 1].elapsed_time(ev[3 * r + 2]) for r in range(reps)) / reps
        return t_topk * 1e-3, t_att * 1e-3

    def free(self):
        del self.pooled, self.q, self.hw, self.qa, self.db
        self.torch.cuda.empty_cache()


def oracle_step_time(dec, budget_s=25.0):
    """The CPU oracle on one full decode step of the same workload: scores of every
    group, top-512 selection and 64-head attention for each sequence, from the
    GPU's pooled keys (rotation set 0).  Rows are processed until the time budget
    is spent; the step time is scaled from the rows done."""
    import oracle

    wl, db = dec.wl, dec.db
    B = wl.batch
    q, hw, qa = wl.q_idx(0, B), wl.head_w(0, B), wl.q_attn(0, B)
    lat = db.host["latent"]
    to = wl.token_offsets
    pooled = []
    for b in range(B):
        pages = db.bt[b, : wl.pages(b)].long()
        pooled.append(dec.pooled[0][pages].reshape(-1, 128)[: wl.groups(b)].cpu().numpy())
    threads = oracle.n_threads()
    t0 = time.perf_counter()
    rows = 0
    for b in range(B):
        S = oracle.scores(q[b], hw[b], pooled[b], threads=threads)
        idx, cnt = oracle.topk(S, 512)
        oracle.attention(qa[b], lat[to[b]: to[b + 1]], wl.lens[b], wl.lens[b] - 1, idx, cnt, 1.0 / math.sqrt(512))
        rows += 1
        if time.perf_counter() - t0 > budget_s:
            break
    spent = time.perf_counter() - t0
    step_s = spent * B / rows
    return {"value": round(1.0 / step_s, 4), "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of {B} sequences of one decode step of {wl.name} (every pooled group scored, "
                      f"top-512 selected, 64-head attention over the selection), scaled to the whole step; "
                      f"scoring spread over {threads} threads, selection and attention on one",
            "seconds": round(spent, 2)}


def bench_prefill(args):
    """Prefill indexer scores of 2048 queries over 262,144 pooled groups (int8 MFMA)."""
    import numpy as np
    import torch

    import harness as H
    import long_context_sparse_indexpool_amd as m
    from synth.configs import workload

    wl = workload(3)
    db = H.make_batch(wl, with_keys=True, with_latent=False, keep_host=False)
    H.run_pool(db)
    del db.keys
    Q = wl.rows
    G = wl.groups(0)
    qd = torch.from_numpy(wl.q_idx()).cuda()
    hwd = torch.from_numpy(wl.head_w()).cuda()
    qpos = torch.from_numpy(wl.row_pos()).cuda()
    sc = torch.empty((Q, G), dtype=torch.int32, device="cuda")
    ws = m.alloc_workspace(256)
    run = lambda: m.isa_indexer_prefill_scores(qd, hwd, qpos, Q, db.pooled, db.seqs, sc, G, ws)
    for _ in range(2):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps * 1e-3
    useful_ops = sum(2 * 32 * 128 * (int(p) // 4 + 1) for p in wl.row_pos())
    dense_ops = 2 * Q * 32 * 128 * G
    # selection over the 2 GiB score matrix
    idx = torch.empty((Q, 512), dtype=torch.int32, device="cuda")
    cnt = torch.empty(Q, dtype=torch.int32, device="cuda")
    m.isa_indexer_topk(None, None, None, None, sc, Q, G, 512, idx, cnt, None, ws)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(3):
        m.isa_indexer_topk(None, None, None, None, sc, Q, G, 512, idx, cnt, None, ws)
    e1.record()
    torch.cuda.synchronize()
    t_sel = e0.elapsed_time(e1) / 3 * 1e-3
    res = {"workload": wl.name, "ms": round(t * 1e3, 4), "useful_TOPS": round(useful_ops / t / 1e12, 1),
           "dense_TOPS": round(dense_ops / t / 1e12, 1), "frac_int8_peak": round(dense_ops / t / 1e12 / INT8_PEAK_TOPS, 4),
           "select_ms": round(t_sel * 1e3, 4), "select_GBps": round(2 * Q * G * 4 / t_sel / 1e9, 1)}
    del sc, db
    torch.cuda.empty_cache()
    return res


def bench_pool(dec):
    """isa_indexpool (dynamic scale: amax pass + pool/quantise pass) on the decode workload's keys."""
    import torch

    import harness as H
    import long_context_sparse_indexpool_amd as m

    wl = dec.wl
    keys = H.pool_from_logical(wl, wl.keys_logical(), 256, H.NAN_BF16)
    pooled = torch.empty_like(dec.pooled[0])
    scales = torch.empty(wl.batch, dtype=torch.float32, device="cuda")
    ws = m.alloc_workspace(m.workspace_size(m.ISA_OP_INDEXPOOL, dec.db.seqs))
    w4 = wl.pool_weights()
    out = {}
    for name, flags in (("dynamic", 0), ("given_scale", 1)):
        m.isa_indexpool(keys, w4, dec.db.seqs, scales, pooled, flags, ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            m.isa_indexpool(keys, w4, dec.db.seqs, scales, pooled, flags, ws)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 5 * 1e-3
        alg = wl.total_tokens * 256 + sum(wl.groups(b) for b in range(wl.batch)) * 128
        out[name] = {"ms": round(t * 1e3, 3), "alg_GBps": round(alg / t / 1e9, 1)}
    del keys, pooled
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--primary-only", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (sharding is described in DESIGN.md); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from synth.configs import workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    import long_context_sparse_indexpool_amd as m  # noqa: F401  (fails loudly when libisa.so is missing)

    wl = workload(2)
    dec = Decode(wl, N_POOL_COPIES, N_QSETS, keep_host=not args.no_cpu_baseline)
    sec_per_step = dec.time_steps(args.steps, args.warmup)
    t_topk, t_att = dec.time_kernels(20)
    log(f"{wl.name}: {1 / sec_per_step:.1f} steps/s, indexer {t_topk * 1e6:.1f} us, attention {t_att * 1e6:.1f} us")
    steps_per_s = 1.0 / sec_per_step
    traffic = measured_traffic("k_indexer_decode", wl.name)
    roof = {"kernel": "k_indexer_decode", "bound": "hbm", "achieved": round(dec.bytes_topk / t_topk / 1e9, 1),
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(dec.bytes_topk / t_topk / 1e9 / HBM_PEAK_GBPS, 4),
            "traffic": traffic, "alg_bytes_per_launch": dec.bytes_topk, "avg_launch_us": round(t_topk * 1e6, 2)}
    result = {
        "metric": METRIC, "value": round(steps_per_s, 1), "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(sec_per_step * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8+bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "seq_len": wl.lens[0], "topk_groups": 512,
                   "group_tokens": 4, "indexer_heads": 32, "attention_heads": 64, "latent_dim": 512},
        "achieved_hbm_GBps": round(dec.bytes_step * steps_per_s / 1e9, 1),
        "hbm_frac": round(dec.bytes_step * steps_per_s / 1e9 / HBM_PEAK_GBPS, 4),
        "alg_bytes_per_step": dec.bytes_step,
        "roofline": roof,
        "kernels_us": {"indexer_topk": round(t_topk * 1e6, 2), "sparse_mla": round(t_att * 1e6, 2)},
    }
    if not args.no_cpu_baseline:
        log("oracle baseline")
        result["cpu_baseline"] = oracle_step_time(dec)
        dec.db.host.clear()
    secondary = {}
    if not args.primary_only:
        secondary["indexpool"] = bench_pool(dec)
    dec.free()
    if not args.primary_only:
        for i in (1, 4):
            w = workload(i)
            d = Decode(w, 2, 4)
            s = d.time_steps(50, 5)
            tk, ta = d.time_kernels(10)
            secondary[w.name] = {"steps_per_s": round(1 / s, 1), "ms_per_step": round(s * 1e3, 4),
                                 "achieved_hbm_GBps": round(d.bytes_step / s / 1e9, 1),
                                 "indexer_us": round(tk * 1e6, 2), "sparse_mla_us": round(ta * 1e6, 2),
                                 "alg_bytes_per_step": d.bytes_step}
            d.free()
        secondary["prefill_scores"] = bench_prefill(args)
    result["secondary"] = secondary
    result["env"] = {"device": torch.cuda.get_device_name(0), "torch": torch.__version__,
                     "hip": getattr(torch.version, "hip", None)}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
