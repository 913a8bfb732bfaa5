"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (whole batch per call, scores not requested), against the CPU
oracle.

Decode workloads (8192 tokens; 64 x 131,072; 8 x 1,048,576; 32 ragged paged
sequences up to 2^20; 256 sequences, one of the maximum 2^22 tokens): pooled keys of every sequence within 1 LSB, every score
bit-exact (from a second call that also writes the scores), every selected id
bit-exact, and attention within tolerance for every row.  At 8 x 1,048,576 also
IndexShare: four layers' attention over the same selection in one call, every
row of every layer against the oracle.  The prefill chunk (2048 queries at the
end of one 2^20-token sequence): the mask of every score row, every row's
scores bit-exact and its selected ids against the oracle's top-k of those
scores, and attention on one row of every 16-query block.
"""
import numpy as np
import pytest
import torch

import oracle
from synth.configs import GROUP, SM_SCALE, TOPK_GROUPS, custom, workload

import harness as H

pytestmark = pytest.mark.gpu


def _decode_full(wl, share_layers: int = 0):
    B = wl.batch
    H.log(f"{wl.name}: generating inputs")
    db = H.make_batch(wl, keep_host=True)
    H.run_pool(db)
    H.log(f"{wl.name}: pool parity, {B} sequences")
    H.check_pool(db)

    q, hw = wl.q_idx(0, B), wl.head_w(0, B)
    H.log(f"{wl.name}: top-k as timed (no score output)")
    idx, cnt, _, _ = H.run_topk(db, with_scores=False, q=q, hw=hw)
    _, _, sc, _ = H.run_topk(db, with_scores=True, q=q, hw=hw)
    idx2, cnt2, _, _ = H.run_topk(db, with_scores=False, q=q, hw=hw)
    assert np.array_equal(idx, idx2) and np.array_equal(cnt, cnt2), "selection differs between calls"

    H.log(f"{wl.name}: oracle scores and selection")
    refs = oracle.map_rows(lambda b: H.oracle_scores_for(db, b), range(B))
    for b in range(B):
        G = wl.groups(b)
        assert np.array_equal(sc[b, :G].astype(np.int64), refs[b]), f"scores of sequence {b}"
        H.check_topk_row(refs[b], TOPK_GROUPS, idx[b], int(cnt[b]))

    H.log(f"{wl.name}: attention, {B} rows")
    idx_d = torch.from_numpy(idx).cuda()
    cnt_d = torch.from_numpy(cnt).cuda()
    out, lse = H.run_attention(db, idx_d, cnt_d, TOPK_GROUPS, q=wl.q_attn(0, B))
    qa, lat, to = db.host["q_attn"], db.host["latent"], wl.token_offsets

    def one(b):
        L = wl.lens[b]
        return oracle.attention(qa[b], lat[to[b]: to[b + 1]], L, L - 1, idx[b], int(cnt[b]), SM_SCALE)

    ref_att = oracle.map_rows(one, range(B))
    for b in range(B):
        H.attention_tolerance(out[b], ref_att[b][0], lse[b], ref_att[b][1])
    if share_layers:
        _index_share_full(db, idx, cnt, idx_d, cnt_d, ref_att, share_layers)
        _fp8_full(db, idx, cnt, idx_d, cnt_d)
    H.log(f"{wl.name}: done")


def test_decode_tiles_between_sizes():
    """A batch that makes fewer scoring tiles than CUs at 8192 groups per tile
    (8 x 600,000 tokens: 152 tiles of 8192, 296 of 4096), so the scoring runs
    with the smallest tile that fits one round over the CUs (4736 groups, 256
    tiles, not a power of two): every score and every selected id bit-exact
    against the oracle, with and without the score output."""
    wl = custom("tile4096", 23, [600000] * 8, paged_random=True)
    B = wl.batch
    db = H.make_batch(wl, with_latent=False)
    H.run_pool(db)
    idx, cnt, sc, _ = H.run_topk(db, with_scores=True)
    idx2, cnt2, _, _ = H.run_topk(db, with_scores=False)
    assert np.array_equal(idx, idx2) and np.array_equal(cnt, cnt2), "selection differs with the score output"
    refs = oracle.map_rows(lambda b: H.oracle_scores_for(db, b), range(B))
    for b in range(B):
        G = wl.groups(b)
        assert np.array_equal(sc[b, :G].astype(np.int64), refs[b]), f"scores of sequence {b}"
        H.check_topk_row(refs[b], TOPK_GROUPS, idx[b], int(cnt[b]))


def test_decode_tiles_at_exact_boundaries():
    """Forty sequences of about six 2560-group tiles each (on 256 CUs the
    smallest tile that fits one round: 242 tiles), ending exactly on a tile
    boundary, one group short of it, one group past it (a last tile of a single
    group) and a little further in, with partial last groups; the full pairs of
    tiles move groups between their halves.  Every score and every selected id
    bit-exact against the oracle."""
    T = 2560
    groups = [6 * T, 6 * T - 1, 6 * T + 1, 6 * T - 32, 6 * T - 33, 6 * T - 63] + [6 * T - 64 + 2 * i for i in range(34)]
    lens = [4 * g - (i % 4) for i, g in enumerate(groups)]
    wl = custom("tile_bounds", 41, lens, paged_random=True)
    B = wl.batch
    db = H.make_batch(wl, with_latent=False)
    H.run_pool(db)
    idx, cnt, sc, _ = H.run_topk(db, with_scores=True)
    refs = oracle.map_rows(lambda b: H.oracle_scores_for(db, b), range(B))
    for b in range(B):
        G = wl.groups(b)
        assert np.array_equal(sc[b, :G].astype(np.int64), refs[b]), f"scores of sequence {b} (G = {G})"
        H.check_topk_row(refs[b], TOPK_GROUPS, idx[b], int(cnt[b]))


def _fp8_full(db, idx, cnt, idx_d, cnt_d):
    """FP8 latent cache at full size: the whole pool quantised on the GPU, the
    selected rows' codes and scales bit-exact against the oracle's quantiser, and
    attention over the FP8 cache against the oracle's FP8 attention for every row
    (the oracle runs on the selected rows only: every sequence length is a
    multiple of 4, so each selected group is complete and visible)."""
    wl = db.wl
    B = wl.batch
    H.log(f"{wl.name}: FP8 latent cache")
    codes, scales = H.latent_fp8(db)
    out, lse = H.run_attention_fp8(db, codes, scales, idx_d, cnt_d, TOPK_GROUPS, q=wl.q_attn(0, B))
    lat, to = db.host["latent"], wl.token_offsets
    qa = wl.q_attn(0, B)
    toks, gc, gs = [], [], []
    for b in range(B):
        assert wl.lens[b] % GROUP == 0
        n = int(cnt[b])
        tok = (idx[b, :n].astype(np.int64)[:, None] * GROUP + np.arange(GROUP)).reshape(-1)
        toks.append(tok)
        gc.append(H.logical_rows(db, codes, b, tok))
        gs.append(H.logical_rows(db, scales, b, tok))
    del codes, scales

    def one(b):
        rc, rs = oracle.latent_fp8(lat[to[b] + toks[b]])
        assert np.array_equal(gc[b], rc) and np.array_equal(gs[b], rs), f"codes of sequence {b}"
        n = int(cnt[b])
        return oracle.attention_fp8(qa[b], rc, rs, GROUP * n, GROUP * n - 1, np.arange(n, dtype=np.int32), n,
                                    SM_SCALE)

    ref = oracle.map_rows(one, range(B))
    for b in range(B):
        H.attention_tolerance(out[b], ref[b][0], lse[b], ref[b][1])


def _index_share_full(db, idx, cnt, idx_d, cnt_d, ref0, n):
    """n layers over the same selection in one call, every row of every layer
    against the oracle (layer l's cache is layer 0's with its flipped channels)."""
    from synth.configs import layer_flip_view
    wl = db.wl
    B = wl.batch
    H.log(f"{wl.name}: IndexShare, {n} layers in one call")
    pools = H.layer_latents(db, n)
    res = H.run_attention_shared(db, idx_d, cnt_d, TOPK_GROUPS, pools)
    del pools
    for b in range(B):
        H.attention_tolerance(res[0][0][b], ref0[b][0], res[0][1][b], ref0[b][1])
    lat, to = db.host["latent"], wl.token_offsets
    for layer in range(1, n):
        qa = wl.q_attn(0, B, layer=layer)
        view = layer_flip_view(lat, layer)
        view ^= np.uint16(0x8000)
        try:
            def one(b):
                L = wl.lens[b]
                return oracle.attention(qa[b], lat[to[b]: to[b + 1]], L, L - 1, idx[b], int(cnt[b]), SM_SCALE)
            ref = oracle.map_rows(one, range(B))
        finally:
            view ^= np.uint16(0x8000)
        for b in range(B):
            H.attention_tolerance(res[layer][0][b], ref[b][0], res[layer][1][b], ref[b][1])


def test_full_decode_b1_L8192():
    _decode_full(workload(0))


def test_full_decode_b64_L131072():
    _decode_full(workload(1))


def test_full_decode_b8_L1048576():
    _decode_full(workload(2), share_layers=4)


def test_full_ragged_paged_b32():
    _decode_full(workload(4))


def test_full_decode_max_batch_and_length():
    """The largest sizes the library accepts, in one call: ISA_MAX_BATCH = 256
    sequences, one of them ISA_MAX_SEQ_LEN = 2^22 tokens (128 scoring tiles of
    8192 groups, the per-sequence maximum) and 255 ragged ones of 1..20,000
    tokens, pages placed at random; one attention split per row at this batch.
    Pooled keys, every score and selected id, and every row's attention
    against the oracle."""
    m = H.isa()
    assert m.MAX_BATCH == 256 and m.MAX_SEQ_LEN == 1 << 22
    rng = np.random.default_rng(31)
    lens = [m.MAX_SEQ_LEN] + [int(x) for x in rng.integers(1, 20001, m.MAX_BATCH - 1)]
    _decode_full(custom("max_batch_and_length", 31, lens, paged_random=True))


def test_full_prefill_q2048_L1048576():
    m = H.isa()
    wl = workload(3)
    Q, G, L = wl.rows, wl.groups(0), wl.lens[0]
    H.log(f"{wl.name}: generating inputs")
    db = H.make_batch(wl, keep_host=True)
    H.run_pool(db)
    qh, hwh, qpos = wl.q_idx(), wl.head_w(), wl.row_pos()
    sc = torch.empty((Q, G), dtype=torch.int32, device="cuda")
    ws = m.alloc_workspace(256)
    H.log(f"{wl.name}: prefill scores {Q} x {G}")
    m.isa_indexer_prefill_scores(torch.from_numpy(qh).cuda(), torch.from_numpy(hwh).cuda(),
                                 torch.from_numpy(qpos).cuda(), Q, db.pooled, db.seqs, sc, G, ws)
    torch.cuda.synchronize()
    assert m.isa_device_error(ws) == 0
    # the block-causal mask on every row, at full size: -1 exactly after the query's own group
    last = torch.from_numpy(qpos // 4).cuda().long()
    cols = torch.arange(G, device="cuda")
    masked = cols[None, :] > last[:, None]
    assert bool((sc[masked] == -1).all()), "masked entries must be -1"
    assert bool((sc[~masked] >= 0).all()), "visible entries must be valid scores"
    del masked

    idx = torch.empty((Q, TOPK_GROUPS), dtype=torch.int32, device="cuda")
    cnt = torch.empty(Q, dtype=torch.int32, device="cuda")
    m.isa_indexer_topk(None, None, None, None, sc, Q, G, TOPK_GROUPS, idx, cnt, None, ws)
    torch.cuda.synchronize()
    out, lse = H.run_attention(db, idx, cnt, TOPK_GROUPS, row_seq=np.zeros(Q, np.int32), row_pos=qpos, rows=Q)
    idxh, cnth = idx.cpu().numpy(), cnt.cpu().numpy()

    # every row: scores bit-exact against the oracle, ids against the oracle's
    # top-k of those scores (rows in chunks, so the host holds one chunk)
    k8 = H.pooled_logical(db, 0)
    chunk = 128
    for r0 in range(0, Q, chunk):
        rows = list(range(r0, min(Q, r0 + chunk)))
        H.log(f"{wl.name}: oracle scores and selection of rows {rows[0]}..{rows[-1]}")
        S = sc[rows[0]: rows[-1] + 1].cpu().numpy()

        def one(r):
            ref = oracle.prefill_scores(qh[r], hwh[r], int(qpos[r]), k8)
            assert np.array_equal(S[r - r0].astype(np.int64), ref), f"scores of query {r}"
            H.check_topk_row(ref, TOPK_GROUPS, idxh[r], int(cnth[r]))
            return True

        assert all(oracle.map_rows(one, rows))
        del S
    # attention: one row of every 16-query block, plus the last rows
    att_rows = sorted(set(range(0, Q, 16)) | {1, 2, 3, Q - 2, Q - 1} | set(range(7, Q, 16 * 8)))
    H.log(f"{wl.name}: oracle attention on {len(att_rows)} rows")
    qa, lat = db.host["q_attn"], db.host["latent"]
    ref_att = oracle.map_rows(
        lambda r: oracle.attention(qa[r], lat, L, int(qpos[r]), idxh[r], int(cnth[r]), SM_SCALE), att_rows)
    for j, r in enumerate(att_rows):
        H.attention_tolerance(out[r], ref_att[j][0], lse[r], ref_att[j][1])
    H.log(f"{wl.name}: done")
