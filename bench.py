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
BF16_PEAK_TFLOPS = 2500.0
N_POOL_COPIES = 4
N_QSETS = 16
KERNEL_SOURCES = {
    "k_indexer_score": ["indexer_decode.hip", "select_device.hpp", "isa_common.hpp", "isa_launch.hpp"],
    "k_mla_split": ["mla_decode.hip", "isa_common.hpp", "isa_launch.hpp"],
    "k_mla_combine": ["mla_decode.hip", "isa_common.hpp", "isa_launch.hpp"],
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
        # scoring kernel: 128 B per pooled group of every sequence longer than k groups,
        # plus each sequence's int8 query (32 x 128) and head weights (32)
        self.groups_scored = sum(g for g in G if g > self.k)
        self.bytes_score = 128 * self.groups_scored + B * (32 * 128 + 32)
        self.bytes_topk = self.bytes_score + B * (self.k * 4 + 4)
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

    def time_steps(self, steps, warmup, event_every=0):
        """Seconds per step over exactly `steps` back-to-back steps after `warmup`.
        With event_every = E > 0, also the average durations of the scoring kernel
        and of the attention kernel over the last step of every E of those same
        steps: HIP events that the library attaches to the two dispatches
        (hipExtLaunchKernelGGL, enabled by isa_set_kernel_timer), on the stream
        it launches on.  Each event pair adds a few microseconds to its step, so
        only a sample of the timed steps carries them."""
        torch, m = self.torch, self.m
        for _ in range(warmup):
            self.step()
        evs = {}
        n = steps // event_every if event_every else 0
        if n:
            evs = {k: ([torch.cuda.Event(enable_timing=True) for _ in range(n)],
                       [torch.cuda.Event(enable_timing=True) for _ in range(n)])
                   for k in (m.ISA_TIMER_INDEXER_SCORE, m.ISA_TIMER_MLA_SPLIT)}
            for a, b in evs.values():
                for e in a + b:
                    e.record()  # creates the event
        torch.cuda.synchronize()
        try:
            t0 = time.perf_counter()
            for i in range(steps):
                j = i // event_every if n and i % event_every == event_every - 1 else -1
                for k, (a, b) in evs.items():
                    if j >= 0:
                        m.isa_set_kernel_timer(k, [a[j]], [b[j]])
                self.step()
                if j >= 0:
                    for k in evs:
                        m.isa_set_kernel_timer(k, [], [])
            torch.cuda.synchronize()
            sec = (time.perf_counter() - t0) / steps
        finally:
            for k in evs:
                m.isa_set_kernel_timer(k, [], [])
        if not event_every:
            return sec
        if not n:
            raise ValueError("fewer timed steps than event_every")
        avg = {k: sum(x.elapsed_time(y) for x, y in zip(a, b)) / n * 1e-3 for k, (a, b) in evs.items()}
        return sec, avg[m.ISA_TIMER_INDEXER_SCORE], avg[m.ISA_TIMER_MLA_SPLIT]

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


def bench_index_share(dec, n_layers=4, steps=100, warmup=10):
    """IndexShare on the headline workload: one indexer call and the attention
    of n_layers layers over its selection, (a) in one shared call, (b) as
    n_layers single-layer calls.  Layer l >= 1 has its own query and a latent
    pool of its own (a device copy of layer 0's with sign-flipped channels)."""
    import numpy as np
    import torch

    import harness as H
    from synth.configs import SM_SCALE

    m, wl = dec.m, dec.wl
    B = wl.batch
    pools = H.layer_latents(dec.db, n_layers)
    qs = [torch.from_numpy(wl.q_attn(0, B, layer=l).view(np.int16)).cuda() for l in range(n_layers)]
    outs = [torch.empty((B, 64, 512), dtype=torch.float32, device="cuda") for _ in range(n_layers)]
    lses = [torch.empty((B, 64), dtype=torch.float32, device="cuda") for _ in range(n_layers)]
    ws_sh = m.alloc_workspace(m.workspace_size(m.ISA_OP_SPARSE_MLA, dec.db.seqs, B, n_layers))

    def shared(j):
        dec.topk(j)
        m.isa_sparse_mla_decode_shared(qs, pools, dec.db.seqs, None, None, B, dec.idx, dec.cnt, dec.k, SM_SCALE,
                                       outs, lses, ws_sh)

    def separate(j):
        dec.topk(j)
        for l in range(n_layers):
            m.isa_sparse_mla_decode(qs[l], pools[l], dec.db.seqs, None, None, B, dec.idx, dec.cnt, dec.k, SM_SCALE,
                                    outs[l], lses[l], dec.ws_att)

    res = {"layers": n_layers}
    for name, fn in (("shared", shared), ("separate", separate)):
        for j in range(warmup):
            fn(j)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for j in range(steps):
            fn(j)
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / steps
        res[f"steps_per_s_{name}"] = round(1 / sec, 1)
        res[f"ms_per_step_{name}"] = round(sec * 1e3, 4)
    del pools, qs, outs, lses, ws_sh
    torch.cuda.empty_cache()
    log(f"{wl.name}: IndexShare over {n_layers} layers: {res['steps_per_s_shared']} steps/s in one call, "
        f"{res['steps_per_s_separate']} with separate calls")
    return res


def bench_fp8(dec, steps=100, warmup=10):
    """FP8 latent cache on the headline workload: the whole latent pool quantised
    once (isa_latent_to_fp8, timed), then decode steps with the attention over the
    FP8 cache (512 B + a 4 B scale per token instead of 1 KiB)."""
    import torch

    import harness as H
    from synth.configs import SM_SCALE

    m, wl = dec.m, dec.wl
    B = wl.batch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    codes, scales = H.latent_fp8(dec.db)
    t_q = time.perf_counter() - t0

    def step(j):
        dec.topk(j)
        m.isa_sparse_mla_decode_fp8(dec.qa[j % len(dec.qa)], codes, scales, dec.db.seqs, None, None, B, dec.idx,
                                    dec.cnt, dec.k, SM_SCALE, dec.out, dec.lse, dec.ws_att)

    for j in range(warmup):
        step(j)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(steps):
        step(j)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for j in range(20):
        m.isa_sparse_mla_decode_fp8(dec.qa[j % len(dec.qa)], codes, scales, dec.db.seqs, None, None, B, dec.idx,
                                    dec.cnt, dec.k, SM_SCALE, dec.out, dec.lse, dec.ws_att)
    ev[1].record()
    torch.cuda.synchronize()
    t_att = ev[0].elapsed_time(ev[1]) / 20 * 1e3
    tokens = sum(wl.lens)
    del codes, scales
    torch.cuda.empty_cache()
    res = {"steps_per_s": round(1 / sec, 1), "ms_per_step": round(sec * 1e3, 4), "sparse_mla_us": round(t_att, 2),
           "quantise_ms": round(t_q * 1e3, 2), "quantise_GBps": round(tokens * (1024 + 512 + 4) / t_q / 1e9, 1)}
    log(f"{wl.name}: FP8 latent cache: {res['steps_per_s']} steps/s, attention call {t_att:.1f} us")
    return res


def bench_kda(batch=8, heads=32, reps=200):
    """Linear-attention (KDA) decode step of one layer for `batch` sequences x
    `heads` heads: 32 KiB of bf16 state read and written per head, plus the
    per-token vectors.  Reported as us per step and algorithmic GB/s."""
    import numpy as np
    import torch

    import long_context_sparse_indexpool_amd as m
    from synth.configs import kda_inputs, kda_state
    n = batch * heads
    st = torch.from_numpy(kda_state(7, n).view(np.int16)).cuda()
    q, k, v, alpha, beta = [torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda()
                            for x in kda_inputs(7, n, 0)]
    out = torch.empty((n, 128), dtype=torch.float32, device="cuda")
    ws = m.alloc_workspace(m.workspace_size(m.ISA_OP_KDA_STEP, None))
    for _ in range(10):
        m.isa_kda_decode_step(q, k, v, alpha, beta, st, out, ws)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(reps):
        m.isa_kda_decode_step(q, k, v, alpha, beta, st, out, ws)
    ev[1].record()
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) / reps * 1e3
    nbytes = n * (2 * 128 * 128 * 2 + 3 * 128 * 2 + 128 * 4 + 4 + 128 * 4)
    assert m.isa_device_error(ws) == 0
    log(f"KDA decode step: {n} heads in {us:.2f} us, {nbytes / us / 1e3:.1f} GB/s")
    return {"units": n, "batch": batch, "heads": heads, "us_per_step": round(us, 2),
            "alg_bytes_per_step": nbytes, "alg_GBps": round(nbytes / us / 1e3, 1)}


def bench_append(batch=8, length=1 << 20, reps=200):
    """Decode-time cache maintenance: isa_append_token for a batch of
    `batch` sequences at `length` tokens (one new key and latent row each, the
    token's group re-pooled at a fixed scale).  Only the pages around the new
    tokens are allocated; a call touches ~2.5 KiB per sequence, so it is
    launch- and latency-bound and reported as microseconds per call."""
    import numpy as np
    import torch

    import long_context_sparse_indexpool_amd as m
    B = batch
    pages = B  # one physical page per sequence: the page of the new token
    max_pages = (length + 255) // 256
    bt = torch.full((B, max_pages), 0, dtype=torch.int32)
    bt[:, (length - 1) // 256] = torch.arange(B, dtype=torch.int32)
    bt = bt.cuda()
    seqs = m.Seqs([length] * B, bt, pages)
    keys = torch.zeros((pages, 256, 128), dtype=torch.int16, device="cuda")
    lat = torch.zeros((pages, 256, 512), dtype=torch.int16, device="cuda")
    pooled = torch.zeros((pages, 64, 128), dtype=torch.int8, device="cuda")
    knew = torch.ones((B, 128), dtype=torch.int16, device="cuda")
    lnew = torch.ones((B, 512), dtype=torch.int16, device="cuda")
    sc = torch.ones(B, dtype=torch.float32, device="cuda")
    ws = m.alloc_workspace(m.workspace_size(m.ISA_OP_APPEND_TOKEN, seqs))
    w4 = [0.25, 0.25, 0.25, 0.25]
    for _ in range(10):
        m.isa_append_token(knew, lnew, w4, seqs, sc, keys, lat, pooled, ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        m.isa_append_token(knew, lnew, w4, seqs, sc, keys, lat, pooled, ws)
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / reps * 1e6
    assert m.isa_device_error(ws) == 0
    log(f"append token: batch {B} at {length} tokens: {us:.2f} us per call")
    return {"batch": B, "seq_len": length, "us_per_call": round(us, 2)}


def oracle_step_time(dec, min_s=10.0, budget_s=25.0):
    """The CPU oracle on whole decode steps of the same workload: scores of every
    group, top-512 selection and 64-head attention for each sequence, from the
    GPU's pooled keys (rotation set 0).  Scoring of a sequence is spread over the
    host threads by group ranges; selection and attention run one sequence per
    thread.  Whole steps are repeated until at least `min_s` seconds are spent
    (stopping after the step that passes `budget_s`); per-stage seconds are
    reported beside steps/s."""
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
    t_score = t_sel = t_att = 0.0
    steps = 0
    t0 = time.perf_counter()
    while True:
        a = time.perf_counter()
        S = [oracle.scores(q[b], hw[b], pooled[b], threads=threads) for b in range(B)]
        b_ = time.perf_counter()
        sel = oracle.map_rows(lambda b: oracle.topk(S[b], 512), range(B), threads=threads)
        c = time.perf_counter()
        oracle.map_rows(lambda b: oracle.attention(qa[b], lat[to[b]: to[b + 1]], wl.lens[b], wl.lens[b] - 1,
                                                   sel[b][0], sel[b][1], 1.0 / math.sqrt(512)),
                        range(B), threads=threads)
        d = time.perf_counter()
        t_score, t_sel, t_att = t_score + b_ - a, t_sel + c - b_, t_att + d - c
        steps += 1
        spent = time.perf_counter() - t0
        if spent >= min_s or spent > budget_s:
            break
    return {"value": round(steps / spent, 4), "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{steps} whole decode steps of {wl.name} (every pooled group of the {B} sequences scored, "
                      f"top-512 selected, 64-head attention over the selection); scoring spread over {threads} "
                      f"threads by group range, selection and attention one sequence per thread",
            "seconds": round(spent, 2),
            "stage_seconds_per_step": {"scores": round(t_score / steps, 4), "select": round(t_sel / steps, 4),
                                       "attention": round(t_att / steps, 4)}}


def oracle_single_thread_c0(dec):
    """One decode step of the 8192-token workload through the oracle on one
    thread: pooling of its keys, scores, selection and attention, per stage."""
    import oracle

    wl, db = dec.wl, dec.db
    keys = wl.keys_logical(0)
    t0 = time.perf_counter()
    oracle.pool(keys, wl.pool_weights())
    t1 = time.perf_counter()
    pages = db.bt[0, : wl.pages(0)].long()
    k8 = dec.pooled[0][pages].reshape(-1, 128)[: wl.groups(0)].cpu().numpy()
    q, hw, qa = wl.q_idx(0, 1), wl.head_w(0, 1), wl.q_attn(0, 1)
    t2 = time.perf_counter()
    S = oracle.scores(q[0], hw[0], k8, threads=1)
    idx, cnt = oracle.topk(S, 512)
    t3 = time.perf_counter()
    oracle.attention(qa[0], db.host["latent"], wl.lens[0], wl.lens[0] - 1, idx, cnt, 1.0 / math.sqrt(512))
    t4 = time.perf_counter()
    return {"workload": wl.name, "threads": 1, "pool_s": round(t1 - t0, 4), "scores_select_s": round(t3 - t2, 4),
            "attention_s": round(t4 - t3, 4), "step_s": round(t4 - t2, 4)}


def env_info():
    """Device, software, host CPU and clock facts recorded beside the numbers."""
    import subprocess

    import torch

    p = torch.cuda.get_device_properties(0)
    env = {"device": torch.cuda.get_device_name(0), "arch": getattr(p, "gcnArchName", None),
           "compute_units": p.multi_processor_count, "torch": torch.__version__,
           "hip": getattr(torch.version, "hip", None)}
    try:
        with open("/proc/cpuinfo") as f:
            models = [ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")]
        env["cpu_model"] = models[0] if models else None
        env["cpus_online"] = len(models)
    except OSError:
        env["cpu_model"] = None
    env["cpus_in_affinity"] = len(os.sched_getaffinity(0))
    env["omp_num_threads"] = os.environ.get("OMP_NUM_THREADS")
    try:  # current clock levels as the SMI reports them (read-only query)
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=30)
        env["gpu_clocks"] = [ln.strip() for ln in r.stdout.splitlines() if "clk" in ln.lower() and "level" in ln.lower()]
    except (OSError, subprocess.SubprocessError):
        env["gpu_clocks"] = None
    try:
        r = subprocess.run(["rocm-smi", "--version"], capture_output=True, text=True, timeout=30)
        env["rocm_smi"] = [ln.strip() for ln in r.stdout.splitlines() if ln.strip()][-1:] or None
    except (OSError, subprocess.SubprocessError):
        pass
    return env


def read_ceiling(n_buf=4, buf_bytes=512 << 20, reps=24):
    """Practical HBM read ceiling: isa_read_probe over buffers rotated so that
    none is served from the 256 MB Infinity Cache, timed with HIP events."""
    import torch

    import long_context_sparse_indexpool_amd as m
    bufs = [torch.empty(buf_bytes, dtype=torch.uint8, device="cuda").fill_(i + 1) for i in range(n_buf)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
    for i in range(4):
        m.isa_read_probe(bufs[i % n_buf], sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(reps):
        m.isa_read_probe(bufs[i % n_buf], sink)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps * 1e-3
    m.isa_read_probe(bufs[0], sink, clocks)
    cyc, ticks = [int(x) for x in clocks.cpu()]
    del bufs
    torch.cuda.empty_cache()
    gbps = buf_bytes / t / 1e9
    ghz = cyc / (ticks / 100e6) / 1e9 if ticks else None
    log(f"read ceiling: {gbps:.0f} GB/s ({buf_bytes >> 20} MiB per read, {n_buf} buffers rotated); "
        f"shader clock during the probe {ghz} GHz")
    return {"GBps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4), "bytes_per_read": buf_bytes,
            "buffers_rotated": n_buf,
            "kernel": "isa_read_probe (one workgroup per CU, contiguous shares, wave-wide non-temporal 16-B loads)",
            "shader_clock_GHz_during_probe": round(ghz, 3) if ghz else None}


def bench_prefill(args):
    """Prefill chunk of 2048 queries at the end of one 2^20-token sequence: indexer
    scores over 262,144 pooled groups (int8 MFMA), the selection over the score
    rows, and every row's attention over its selection at its own position."""
    import numpy as np
    import torch

    import harness as H
    import long_context_sparse_indexpool_amd as m
    from synth.configs import SM_SCALE, workload

    wl = workload(3)
    db = H.make_batch(wl, with_keys=True, with_latent=True, keep_host=False)
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
    # steady state: the first launches run while the shader clock is still
    # settling (their duration falls over the first few calls), so five
    # warmup launches, then the median of three groups of five
    for _ in range(5):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps, groups = 5, []
    for _ in range(3):
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        groups.append(e0.elapsed_time(e1) / reps * 1e-3)
    t = sorted(groups)[1]
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
    # attention: every query row over its selection, token-causal at its position
    qa = torch.from_numpy(wl.q_attn(0, Q).view(np.int16)).cuda()
    out = torch.empty((Q, 64, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((Q, 64), dtype=torch.float32, device="cuda")
    rseq = torch.zeros(Q, dtype=torch.int32, device="cuda")
    rpos = qpos.to(torch.int32)
    wsa = m.alloc_workspace(m.workspace_size(m.ISA_OP_SPARSE_MLA, db.seqs, Q))
    run_att = lambda: m.isa_sparse_mla_decode(qa, db.latent, db.seqs, rseq, rpos, Q, idx, cnt, 512, SM_SCALE, out,
                                              lse, wsa)
    run_att()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(3):
        run_att()
    e1.record()
    torch.cuda.synchronize()
    t_att = e0.elapsed_time(e1) / 3 * 1e-3
    pos = wl.row_pos()
    cnt_h = cnt.cpu().numpy().astype(np.int64)
    # tokens attended per row: the selected groups' tokens up to the row's position (selected groups
    # lie at or before the row's own group, so only that group can be partly visible)
    idx_h = idx.cpu().numpy()
    toks = 0
    for r in range(Q):
        g = idx_h[r, : cnt_h[r]].astype(np.int64)
        toks += int(np.minimum(4, pos[r] + 1 - 4 * g).clip(0).sum())
    att_bytes = toks * 1024 + Q * (64 * 512 * 2 + 64 * 512 * 4 + 64 * 4)
    att_flops = 4 * 64 * 512 * toks
    res = {"workload": wl.name, "ms": round(t * 1e3, 4), "ms_groups": [round(x * 1e3, 4) for x in groups], "useful_TOPS": round(useful_ops / t / 1e12, 1),
           "dense_TOPS": round(dense_ops / t / 1e12, 1), "frac_int8_peak": round(dense_ops / t / 1e12 / INT8_PEAK_TOPS, 4),
           "select_ms": round(t_sel * 1e3, 4), "select_GBps": round(2 * Q * G * 4 / t_sel / 1e9, 1),
           "attention_ms": round(t_att * 1e3, 4), "attention_tokens": toks,
           "attention_GBps": round(att_bytes / t_att / 1e9, 1),
           "attention_frac_bf16_peak": round(att_flops / t_att / 1e12 / BF16_PEAK_TFLOPS, 4)}
    del sc, db, out, qa
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


COPY_BYTES = 1 << 30  # plain device copy used to calibrate the HBM byte counters


def traffic_run(index=2, steps=5):
    """Workload for the counter passes: a few decode steps of a decode workload
    (default the 8 x 1M one), then a plain 1 GiB device-to-device copy three
    times (known bytes: 1 GiB read and 1 GiB written per copy), which calibrates
    FETCH_SIZE / WRITE_SIZE."""
    import torch

    from synth.configs import workload

    torch.cuda.set_device(0)
    dec = Decode(workload(index), N_POOL_COPIES, N_QSETS)
    for _ in range(3 + steps):
        dec.step()
    torch.cuda.synchronize()
    dec.free()
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("traffic run done")


def _counter_rows(path):
    """(kernel name, counter, value) of every dispatch in a rocprofv3 counter CSV."""
    import csv

    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            out.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"]), r.get("Dispatch_Id")))
    return out


def summarize_traffic(fetch_csv, write_csv, kernel="k_indexer_score", workload_name="decode_b8_L1048576"):
    """HBM bytes per launch of `kernel` from a FETCH_SIZE pass and a WRITE_SIZE pass
    (KiB per dispatch), each scaled by what the same counter reads for the 1 GiB
    copy; writes profiles/traffic_<kernel>_<workload>.json."""
    def per_dispatch(rows, counter, pred):
        vals = {}
        for name, c, v, d in rows:
            if c.startswith(counter) and pred(name):
                vals[d] = vals.get(d, 0.0) + v
        return sorted(vals.values())

    is_kernel = lambda n: f"isa::{kernel}" in n or n.startswith(kernel)
    is_copy = lambda n: "copyBuffer" in n  # torch's device-to-device copy_ is a runtime blit
    fr, wr = _counter_rows(fetch_csv), _counter_rows(write_csv)
    f_k, w_k = per_dispatch(fr, "FETCH_SIZE", is_kernel), per_dispatch(wr, "WRITE_SIZE", is_kernel)
    f_c, w_c = per_dispatch(fr, "FETCH_SIZE", is_copy), per_dispatch(wr, "WRITE_SIZE", is_copy)
    if not (f_k and w_k and f_c and w_c):
        raise SystemExit(f"missing dispatches: {len(f_k)} {len(w_k)} {len(f_c)} {len(w_c)}")
    med = lambda v: v[len(v) // 2]
    copy_fetch, copy_write = max(f_c) * 1024, max(w_c) * 1024  # the 1 GiB copies are the largest copy dispatches
    ff, wf = copy_fetch / COPY_BYTES, copy_write / COPY_BYTES
    fetch_b, write_b = med(f_k) * 1024, med(w_k) * 1024
    d = {"kernel": kernel, "workload": workload_name, "source_hash": source_hash(kernel),
         "fetch_kib_per_launch": med(f_k), "write_kib_per_launch": med(w_k), "launches": len(f_k),
         "copy_bytes": COPY_BYTES, "copy_fetch_kib": copy_fetch / 1024, "copy_write_kib": copy_write / 1024,
         "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
         "hbm_bytes_per_launch": int(fetch_b / ff + write_b / wf)}
    out = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload_name}.json")
    with open(out, "w") as f:
        json.dump(d, f, indent=1)
    print(json.dumps(d))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--primary-only", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-run", action="store_true", help="workload for the rocprofv3 counter passes")
    ap.add_argument("--traffic-workload", type=int, default=2, metavar="N",
                    help="decode workload of --traffic-run / --summarize-traffic (0, 1, 2 or 4)")
    ap.add_argument("--traffic-kernel", default="k_indexer_score",
                    help="kernel whose bytes --summarize-traffic extracts")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the prefill scoring measurement (for profiling that kernel alone)")
    ap.add_argument("--decode-workload", type=int, default=None, metavar="N",
                    help="only the decode steps of workload N (0, 1, 2 or 4), e.g. to profile a secondary line")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_k_indexer_score_*.json from two counter CSVs (no GPU)")
    args = ap.parse_args()
    if args.summarize_traffic:
        from synth.configs import workload
        summarize_traffic(*args.summarize_traffic, kernel=args.traffic_kernel,
                          workload_name=workload(args.traffic_workload).name)
        return
    if args.traffic_run:
        traffic_run(args.traffic_workload)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (a decode batch would shard by "
              "sequence with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from synth.configs import workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    import long_context_sparse_indexpool_amd as m  # noqa: F401  (fails loudly when libisa.so is missing)
    if args.prefill_only:
        print(json.dumps({"prefill_scores": bench_prefill(args)}), flush=True)
        return
    if args.decode_workload is not None:
        w = workload(args.decode_workload)
        assert w.kind == "decode", "--decode-workload takes a decode workload"
        d = Decode(w, N_POOL_COPIES, N_QSETS)
        s = d.time_steps(args.steps, args.warmup)
        tk, ta = d.time_kernels(10)
        print(json.dumps({w.name: {"steps_per_s": round(1 / s, 1), "ms_per_step": round(s * 1e3, 4),
                                   "achieved_hbm_GBps": round(d.bytes_step / s / 1e9, 1),
                                   "indexer_us": round(tk * 1e6, 2), "sparse_mla_us": round(ta * 1e6, 2)}}),
              flush=True)
        d.free()
        return

    env = env_info()
    wl = workload(2)
    dec = Decode(wl, N_POOL_COPIES, N_QSETS, keep_host=not args.no_cpu_baseline)
    # the timed region (value): exactly `steps` steps, no instrumentation;
    # then the same number of steps again with dispatch events on the scoring
    # and attention kernels of every step, which give the kernels' durations
    # (an event pair adds a few microseconds to its step, so those steps are
    # not the ones the value is taken from)
    sec_per_step = dec.time_steps(args.steps, args.warmup)
    sec_events, t_score, t_split = dec.time_steps(args.steps, 0, event_every=1)
    t_topk, t_att = dec.time_kernels(20)
    # the read-ceiling probe (about 0.1 s of streaming) runs after the timed
    # steps: a saturating stream leaves the shader clock lower for a while, which
    # the latency-bound kernels after the scorer would feel
    ceiling = read_ceiling()
    log(f"{wl.name}: {1 / sec_per_step:.1f} steps/s ({1 / sec_events:.1f} with kernel events); scoring kernel "
        f"{t_score * 1e6:.1f} us, attention kernel {t_split * 1e6:.1f} us; indexer call {t_topk * 1e6:.1f} us, "
        f"attention call {t_att * 1e6:.1f} us")
    steps_per_s = 1.0 / sec_per_step
    traffic = measured_traffic("k_indexer_score", wl.name)
    achieved = dec.bytes_score / t_score / 1e9
    roof = {"kernel": "k_indexer_score", "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
            "alg_bytes_per_launch": dec.bytes_score, "groups_per_launch": dec.groups_scored,
            "alg_bytes_per_group": 128, "avg_launch_us": round(t_score * 1e6, 2),
            "event_samples": args.steps,
            "frac_of_read_ceiling": round(achieved / ceiling["GBps"], 4)}
    result = {
        "metric": METRIC, "value": round(steps_per_s, 1), "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(sec_per_step * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8+bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "seq_len": wl.lens[0], "topk_groups": 512,
                   "group_tokens": 4, "indexer_heads": 32, "attention_heads": 64, "latent_dim": 512},
        "achieved_hbm_GBps": round(dec.bytes_step * steps_per_s / 1e9, 1),
        "hbm_frac": round(dec.bytes_step * steps_per_s / 1e9 / HBM_PEAK_GBPS, 4),
        "alg_bytes_per_step": dec.bytes_step,
        "steps_per_s_with_kernel_events": round(1.0 / sec_events, 1),
        "roofline": roof,
        "read_ceiling": ceiling,
        "kernels_us": {"k_indexer_score": round(t_score * 1e6, 2), "k_mla_split": round(t_split * 1e6, 2),
                       "isa_indexer_topk_call": round(t_topk * 1e6, 2),
                       "isa_sparse_mla_decode_call": round(t_att * 1e6, 2)},
    }
    if not args.no_cpu_baseline:
        log("oracle baseline")
        result["cpu_baseline"] = oracle_step_time(dec)
        dec.db.host.clear()
    secondary = {}
    if not args.primary_only:
        secondary["indexpool"] = bench_pool(dec)
        secondary["index_share"] = bench_index_share(dec)
        secondary["append_token"] = bench_append()
        secondary["fp8_latent"] = bench_fp8(dec)
        secondary["kda_decode"] = bench_kda()
    dec.free()
    if not args.primary_only:
        for i in (0, 1, 4):
            w = workload(i)
            d = Decode(w, N_POOL_COPIES, N_QSETS, keep_host=(i == 0 and not args.no_cpu_baseline))
            s_ = d.time_steps(100, 10)
            tk, ta = d.time_kernels(10)
            line = {"steps_per_s": round(1 / s_, 1), "ms_per_step": round(s_ * 1e3, 4),
                    "achieved_hbm_GBps": round(d.bytes_step / s_ / 1e9, 1),
                    "hbm_frac": round(d.bytes_step / s_ / 1e9 / HBM_PEAK_GBPS, 4),
                    "indexer_us": round(tk * 1e6, 2), "sparse_mla_us": round(ta * 1e6, 2),
                    "alg_bytes_per_step": d.bytes_step, "pooled_copies_rotated": N_POOL_COPIES,
                    "query_sets_rotated": N_QSETS}
            if i == 0:
                line["note"] = "2.56 MB per step: launch- and latency-bound, no roofline claim"
                if not args.no_cpu_baseline:
                    result["cpu_baseline"]["single_thread_" + w.name] = oracle_single_thread_c0(d)
            if i == 1:
                line["fp8_latent"] = bench_fp8(d)
                line["fp8_latent"]["sparse_mla_us_bf16"] = line["sparse_mla_us"]
            secondary[w.name] = line
            d.free()
        secondary["prefill_scores"] = bench_prefill(args)
    result["secondary"] = secondary
    result["env"] = env
    if "cpu_baseline" in result:
        result["cpu_baseline"]["cpu_model"] = env.get("cpu_model")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
