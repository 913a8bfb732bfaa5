"""isa_indexer_topk_noalloc -- the decode-mode top-k on the library's own device
scratch, for callers that cannot allocate -- against isa_indexer_topk on the
same inputs, through the C ABI: calls in a row on one GPU (8 sequences of 2^20
tokens, then a smaller ragged batch with a dense sequence, then saturated keys
whose scores overflow INT32_MAX), each compared bit for bit (selected ids,
counts, scores, device error bits); and a batch larger than the array is
rejected before anything is enqueued.
"""
import numpy as np
import pytest
import torch

import synth
from synth.configs import IDX_DIM, IDX_HEADS, TOPK_GROUPS, custom

import harness as H

pytestmark = pytest.mark.gpu


def _batch(name, seed, lens, saturated=False):
    m = H.isa()
    wl = custom(name, seed, lens, paged_random=True)
    bt = torch.from_numpy(wl.block_table()).cuda()
    db = H.DeviceBatch(wl, m.Seqs(wl.lens, bt, wl.num_pages), bt)
    if saturated:
        db.pooled = torch.full((wl.num_pages, 64, IDX_DIM), 127, dtype=torch.int8, device="cuda")
    else:
        db.pooled = torch.from_numpy(synth.uniform_i8(seed, 40, (wl.num_pages, 64, IDX_DIM), -127, 127)).cuda()
    return db


def _compare(db, seed, saturated=False):
    m = H.isa()
    B = db.wl.batch
    if saturated:
        q = np.full((B, IDX_HEADS, IDX_DIM), 127, np.int8)
        hw = np.full((B, IDX_HEADS), 64, np.int8)
    else:
        q = synth.uniform_i8(seed, 3, (B, IDX_HEADS, IDX_DIM), -127, 127)
        hw = synth.uniform_i8(seed, 4, (B, IDX_HEADS), 0, 64)
    ws = m.alloc_workspace(m.workspace_size(m.ISA_OP_INDEXER_TOPK, db.seqs))
    idx1, cnt1, sc1 = H.topk_into(db, ws, q, hw, with_scores=True)
    err1 = m.isa_device_error(ws)
    ld = sc1.shape[1]
    idx2 = torch.full((B, TOPK_GROUPS), -7, dtype=torch.int32, device="cuda")
    cnt2 = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    sc2 = torch.full((B, ld), -7, dtype=torch.int32, device="cuda")
    err2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    m.isa_indexer_topk_noalloc(torch.from_numpy(q).cuda(), torch.from_numpy(hw).cuda(), db.pooled, db.seqs,
                               TOPK_GROUPS, idx2, cnt2, sc2, ld, err2)
    torch.cuda.synchronize()
    assert np.array_equal(idx2.cpu().numpy(), idx1), f"{db.wl.name}: selected ids differ"
    assert np.array_equal(cnt2.cpu().numpy(), cnt1), f"{db.wl.name}: counts differ"
    for b in range(B):
        G = db.wl.groups(b)
        assert np.array_equal(sc2.cpu().numpy()[b, :G], sc1[b, :G]), f"{db.wl.name}: scores of sequence {b} differ"
    assert int(err2.item()) & 0xFFFFFFFF == err1, f"{db.wl.name}: error bits {int(err2.item()):#x} vs {err1:#x}"
    # and without the score output, as a serving loop would call it
    idx3 = torch.full((B, TOPK_GROUPS), -7, dtype=torch.int32, device="cuda")
    cnt3 = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    m.isa_indexer_topk_noalloc(torch.from_numpy(q).cuda(), torch.from_numpy(hw).cuda(), db.pooled, db.seqs,
                               TOPK_GROUPS, idx3, cnt3, None, 0, err2)
    torch.cuda.synchronize()
    assert np.array_equal(idx3.cpu().numpy(), idx1) and np.array_equal(cnt3.cpu().numpy(), cnt1)
    return err1


def test_noalloc_topk_matches_workspace_topk():
    m = H.isa()
    assert _compare(_batch("noalloc_8x1M", 81, [1 << 20] * 8), 81) == 0
    assert _compare(_batch("noalloc_small", 82, [20000, 3000, 700]), 82) == 0
    assert _compare(_batch("noalloc_overflow", 83, [9000, 2100], saturated=True), 83, saturated=True) == \
        m.DERR_SCORE_OVERFLOW


def test_noalloc_topk_rejects_batches_beyond_its_scratch():
    """16 sequences of 2^20 tokens need 512 scoring tiles, more than the
    array's 384: ISA_ERR_UNSUPPORTED from the host checks, nothing enqueued."""
    m = H.isa()
    B, L = 16, 1 << 20
    bt = torch.zeros((B, L // 256), dtype=torch.int32, device="cuda")
    seqs = m.Seqs([L] * B, bt, L // 256)
    assert m.workspace_size(m.ISA_OP_INDEXER_TOPK, seqs) > m.NOALLOC_TOPK_BYTES
    small = torch.zeros((1, 64, IDX_DIM), dtype=torch.int8, device="cuda")
    q = torch.zeros((B, IDX_HEADS, IDX_DIM), dtype=torch.int8, device="cuda")
    hw = torch.zeros((B, IDX_HEADS), dtype=torch.int8, device="cuda")
    idx = torch.zeros((B, TOPK_GROUPS), dtype=torch.int32, device="cuda")
    cnt = torch.zeros(B, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(m.IsaError) as e:
        m.isa_indexer_topk_noalloc(q, hw, small, seqs, TOPK_GROUPS, idx, cnt, None, 0, err)
    assert e.value.status == m.ISA_ERR_UNSUPPORTED
