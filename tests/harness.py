"""Shared plumbing of the GPU parity tests: seeded inputs -> device page pools ->
the C ABI (through the binding) -> host copies, plus the oracle side.

Only tests (and the smoke check / benchmark) use this module.  The oracle and
the GPU library never meet here except through the same seeded input bytes.
"""
from __future__ import annotations

import math
import sys
import time
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

import oracle
import synth
from synth.configs import (ATT_HEADS, GROUP, IDX_DIM, IDX_HEADS, LAT_DIM, PAGE_GROUPS, PAGE_TOKENS, SM_SCALE,
                           TOPK_GROUPS, Workload)

NAN_BF16 = 0x7FC0  # padding of unused page rows: any read of it would poison the result


def log(msg: str) -> None:
    print(f"[harness {time.strftime('%H:%M:%S')}] {msg}", flush=True)


def isa():
    import long_context_sparse_indexpool_amd as m
    return m


@dataclass
class DeviceBatch:
    wl: Workload
    seqs: object
    bt: torch.Tensor
    keys: Optional[torch.Tensor] = None     # int16 [pages,256,128]
    latent: Optional[torch.Tensor] = None   # int16 [pages,256,512]
    pooled: Optional[torch.Tensor] = None   # int8 [pages,64,128]
    scales: Optional[torch.Tensor] = None
    host: Dict[str, np.ndarray] = field(default_factory=dict)


def pool_from_logical(wl: Workload, logical: np.ndarray, rows_per_page: int, pad) -> torch.Tensor:
    """Host logical rows -> device page pool (identity layouts upload without a copy)."""
    D = logical.shape[1]
    if wl.is_identity_dense() and rows_per_page == PAGE_TOKENS:
        t = torch.from_numpy(logical.view(np.int16) if logical.dtype == np.uint16 else logical)
        return t.reshape(wl.num_pages, rows_per_page, D).cuda()
    pool = wl.scatter_pages(logical, rows_per_page, pad)
    return torch.from_numpy(pool.view(np.int16) if pool.dtype == np.uint16 else pool).cuda()


def make_batch(wl: Workload, with_keys=True, with_latent=True, keep_host=True) -> DeviceBatch:
    m = isa()
    bt = torch.from_numpy(wl.block_table()).cuda()
    seqs = m.Seqs(wl.lens, bt, wl.num_pages)
    db = DeviceBatch(wl, seqs, bt)
    if with_keys:
        keys = wl.keys_logical()
        if keep_host:
            db.host["keys"] = keys
        db.keys = pool_from_logical(wl, keys, PAGE_TOKENS, NAN_BF16)
    if with_latent:
        lat = wl.latent_logical()
        if keep_host:
            db.host["latent"] = lat
        db.latent = pool_from_logical(wl, lat, PAGE_TOKENS, NAN_BF16)
    return db


def run_pool(db: DeviceBatch, flags: int = 0, scales_in: Optional[np.ndarray] = None) -> None:
    m = isa()
    wl = db.wl
    db.pooled = torch.zeros((wl.num_pages, PAGE_GROUPS, IDX_DIM), dtype=torch.int8, device="cuda")
    if scales_in is not None:
        db.scales = torch.from_numpy(np.asarray(scales_in, np.float32)).cuda()
    else:
        db.scales = torch.zeros(wl.batch, dtype=torch.float32, device="cuda")
    ws = m.alloc_workspace(m.workspace_size(m.ISA_OP_INDEXPOOL, db.seqs))
    m.isa_indexpool(db.keys, wl.pool_weights(), db.seqs, db.scales, db.pooled, flags, ws)
    torch.cuda.synchronize()
    err = m.isa_device_error(ws)
    assert err == 0, f"device error word {err:#x}"


def pooled_logical(db: DeviceBatch, b: int) -> np.ndarray:
    """GPU pooled keys of sequence b in logical group order (host int8 [G,128])."""
    wl = db.wl
    G = wl.groups(b)
    pages = db.bt[b, : wl.pages(b)].long()
    return db.pooled[pages].reshape(-1, IDX_DIM)[:G].cpu().numpy()


def run_topk(db: DeviceBatch, k: int = TOPK_GROUPS, with_scores: bool = True, q=None, hw=None):
    m = isa()
    wl = db.wl
    B = wl.batch
    qh = wl.q_idx() if q is None else q
    hwh = wl.head_w() if hw is None else hw
    db.host["q_idx"], db.host["head_w"] = qh, hwh
    qd = torch.from_numpy(qh).cuda()
    hwd = torch.from_numpy(hwh).cuda()
    Gmax = max(wl.groups(b) for b in range(B))
    ld = (Gmax + 3) // 4 * 4
    idx = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((B, ld), -7, dtype=torch.int32, device="cuda") if with_scores else None
    ws = m.alloc_workspace(m.workspace_size(m.ISA_OP_INDEXER_TOPK, db.seqs))
    m.isa_indexer_topk(qd, hwd, db.pooled, db.seqs, None, B, ld, k, idx, cnt, sc, ws)
    torch.cuda.synchronize()
    err = m.isa_device_error(ws)
    assert err == 0, f"device error word {err:#x}"
    return idx.cpu().numpy(), cnt.cpu().numpy(), (sc.cpu().numpy() if sc is not None else None), ws


def topk_into(db: DeviceBatch, ws: torch.Tensor, q: np.ndarray, hw: np.ndarray, k: int = TOPK_GROUPS,
              with_scores: bool = False):
    """isa_indexer_topk (decode mode) on a caller-provided workspace; host (idx, cnt, scores or None)."""
    m = isa()
    B = db.wl.batch
    Gmax = max(db.wl.groups(b) for b in range(B))
    ld = (Gmax + 3) // 4 * 4
    idx = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((B, ld), -7, dtype=torch.int32, device="cuda") if with_scores else None
    m.isa_indexer_topk(torch.from_numpy(q).cuda(), torch.from_numpy(hw).cuda(), db.pooled, db.seqs, None, B, ld, k,
                       idx, cnt, sc, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy(), (sc.cpu().numpy() if sc is not None else None)


def run_attention(db: DeviceBatch, idx: torch.Tensor, cnt: torch.Tensor, k: int, q=None, row_seq=None,
                  row_pos=None, rows=None):
    m = isa()
    wl = db.wl
    rows = wl.batch if rows is None else rows
    qh = wl.q_attn(0, rows) if q is None else q
    db.host["q_attn"] = qh
    qd = torch.from_numpy(qh.view(np.int16)).cuda()
    out = torch.full((rows, ATT_HEADS, LAT_DIM), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((rows, ATT_HEADS), float("nan"), dtype=torch.float32, device="cuda")
    rs = None if row_seq is None else torch.from_numpy(np.asarray(row_seq, np.int32)).cuda()
    rp = None if row_pos is None else torch.from_numpy(np.asarray(row_pos, np.int32)).cuda()
    ws = m.alloc_workspace(m.workspace_size(m.ISA_OP_SPARSE_MLA, db.seqs, rows))
    m.isa_sparse_mla_decode(qd, db.latent, db.seqs, rs, rp, rows, idx, cnt, k, SM_SCALE, out, lse, ws)
    torch.cuda.synchronize()
    err = m.isa_device_error(ws)
    assert err == 0, f"device error word {err:#x}"
    return out.cpu().numpy(), lse.cpu().numpy()


def layer_latents(db: DeviceBatch, n_layers: int):
    """Latent pools of layers 0..n_layers-1 sharing one selection: layer 0 is the
    batch's pool, layer l a device copy with the sign bit of its flipped
    channels set (the input recipe for shared layers)."""
    from synth.configs import layer_flip_view
    pools = [db.latent]
    for layer in range(1, n_layers):
        p = db.latent.clone()
        layer_flip_view(p, layer).bitwise_xor_(-32768)
        pools.append(p)
    return pools


def run_attention_shared(db: DeviceBatch, idx: torch.Tensor, cnt: torch.Tensor, k: int, pools, rows=None):
    """isa_sparse_mla_decode_shared over len(pools) layers (queries from the
    generator's per-layer tensors); returns per-layer (out, lse) on the host."""
    m = isa()
    wl = db.wl
    rows = wl.batch if rows is None else rows
    n = len(pools)
    qs = [torch.from_numpy(wl.q_attn(0, rows, layer=l).view(np.int16)).cuda() for l in range(n)]
    outs = [torch.full((rows, ATT_HEADS, LAT_DIM), float("nan"), dtype=torch.float32, device="cuda")
            for _ in range(n)]
    lses = [torch.full((rows, ATT_HEADS), float("nan"), dtype=torch.float32, device="cuda") for _ in range(n)]
    ws = m.alloc_workspace(m.workspace_size(m.ISA_OP_SPARSE_MLA, db.seqs, rows, n))
    m.isa_sparse_mla_decode_shared(qs, pools, db.seqs, None, None, rows, idx, cnt, k, SM_SCALE, outs, lses, ws)
    torch.cuda.synchronize()
    err = m.isa_device_error(ws)
    assert err == 0, f"device error word {err:#x}"
    return [(o.cpu().numpy(), l.cpu().numpy()) for o, l in zip(outs, lses)]


def latent_fp8(db: DeviceBatch):
    """isa_latent_to_fp8 of the batch's latent pool -> (codes, row_scales) device pools."""
    m = isa()
    wl = db.wl
    codes = torch.zeros((wl.num_pages, PAGE_TOKENS, LAT_DIM), dtype=torch.uint8, device="cuda")
    scales = torch.full((wl.num_pages, PAGE_TOKENS), float("nan"), dtype=torch.float32, device="cuda")
    ws = m.alloc_workspace(m.workspace_size(m.ISA_OP_LATENT_FP8, db.seqs))
    m.isa_latent_to_fp8(db.latent, db.seqs, codes, scales, ws)
    torch.cuda.synchronize()
    err = m.isa_device_error(ws)
    assert err == 0, f"device error word {err:#x}"
    return codes, scales


def logical_rows(db: DeviceBatch, pool: torch.Tensor, b: int, tokens: np.ndarray) -> np.ndarray:
    """Rows of a token-paged device pool for the given tokens of sequence b (host)."""
    bt = db.bt[b].long()
    t = torch.from_numpy(np.asarray(tokens, np.int64)).cuda()
    return pool[bt[t // PAGE_TOKENS], t % PAGE_TOKENS].cpu().numpy()


def run_attention_fp8(db: DeviceBatch, codes, scales, idx: torch.Tensor, cnt: torch.Tensor, k: int, q=None,
                      rows=None):
    m = isa()
    wl = db.wl
    rows = wl.batch if rows is None else rows
    qh = wl.q_attn(0, rows) if q is None else q
    qd = torch.from_numpy(qh.view(np.int16)).cuda()
    out = torch.full((rows, ATT_HEADS, LAT_DIM), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((rows, ATT_HEADS), float("nan"), dtype=torch.float32, device="cuda")
    ws = m.alloc_workspace(m.workspace_size(m.ISA_OP_SPARSE_MLA, db.seqs, rows))
    m.isa_sparse_mla_decode_fp8(qd, codes, scales, db.seqs, None, None, rows, idx, cnt, k, SM_SCALE, out, lse, ws)
    torch.cuda.synchronize()
    err = m.isa_device_error(ws)
    assert err == 0, f"device error word {err:#x}"
    return out.cpu().numpy(), lse.cpu().numpy()


# ------------------------------------------------------------------ comparisons
def check_pool(db: DeviceBatch, bs=None):
    """GPU pooled keys within 1 LSB of the oracle's, scale within 1e-6 relative."""
    wl = db.wl
    keys = db.host["keys"]
    to = wl.token_offsets
    w4 = wl.pool_weights()
    scales = db.scales.cpu().numpy()
    bs = range(wl.batch) if bs is None else bs

    def one(b):
        k8, scale, _, _ = oracle.pool(keys[to[b]: to[b + 1]], w4)
        got = pooled_logical(db, b)
        d = np.abs(got.astype(np.int16) - k8.astype(np.int16))
        return b, int(d.max()), float(abs(scales[b] - scale) / scale), float((d > 0).mean())

    res = oracle.map_rows(one, bs)
    for b, dmax, srel, frac in res:
        assert dmax <= 1, f"seq {b}: pooled differs by {dmax} LSB"
        assert srel <= 1e-6, f"seq {b}: scale relative error {srel}"
    return res


def oracle_scores_for(db: DeviceBatch, b: int) -> np.ndarray:
    return oracle.scores(db.host["q_idx"][b], db.host["head_w"][b], pooled_logical(db, b))


def check_topk_row(S: np.ndarray, k: int, idx_row: np.ndarray, cnt: int):
    ridx, rcnt = oracle.topk(S, k)
    assert cnt == rcnt, f"count {cnt} != oracle {rcnt}"
    assert np.array_equal(idx_row, ridx), "selected ids differ from the oracle"


def attention_tolerance(out: np.ndarray, ref: np.ndarray, lse=None, ref_lse=None):
    """max-abs <= 2e-2 and relative L2 <= 1e-3 (and |d lse| <= 1e-3 where finite),
    the same bound for every row whatever its latent values."""
    d = out.astype(np.float64) - ref
    mx = float(np.max(np.abs(d))) if d.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(d) / nrm) if nrm > 0 else float(np.linalg.norm(d))
    assert np.all(np.isfinite(out)), "non-finite attention output"
    assert mx <= 2e-2, f"max-abs error {mx}"
    assert rel <= 1e-3, f"relative L2 error {rel}"
    dl = 0.0
    if lse is not None:
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isfinite(lse), fin)
        if fin.any():
            dl = float(np.max(np.abs(lse[fin] - ref_lse[fin])))
        assert dl <= 1e-3, f"lse error {dl}"
    return mx, rel, dl
