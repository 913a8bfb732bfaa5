"""GPU parity of the HIP path against the CPU oracle on small seeded inputs that
still span several work tiles, ragged tails, the dense fallback and ties.

Bars: pooled keys within 1 int8 LSB and scales within 1e-6 relative; indexer
scores and selected ids bit-exact; attention max-abs <= 2e-2, relative L2 <=
1e-3, |d lse| <= 1e-3.  Every case runs through the C ABI.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth.configs import IDX_DIM, LAT_DIM, SM_SCALE, _to_bf16_bits, custom

import harness as H

pytestmark = pytest.mark.gpu

RAGGED = [1, 2, 3, 4, 5, 255, 256, 257, 1001, 2047, 2048, 2049, 2052, 4099, 8192, 8195, 9000, 20003]


@pytest.fixture(scope="module")
def ragged_batch():
    H.log("ragged batch: pool")
    wl = custom("ragged", 11, RAGGED, paged_random=True)
    db = H.make_batch(wl)
    H.run_pool(db)
    return db


def test_library_loads_on_gpu():
    m = H.isa()
    assert "gfx950" in m.version()


def test_pool_parity_ragged(ragged_batch):
    res = H.check_pool(ragged_batch)
    assert len(res) == len(RAGGED)


def test_pool_given_scale(ragged_batch):
    db = ragged_batch
    wl = db.wl
    given = db.scales.cpu().numpy() * np.float32(0.5)  # half the dynamic scale: values clamp at +-127
    db2 = H.DeviceBatch(wl, db.seqs, db.bt, keys=db.keys, host=db.host)
    H.run_pool(db2, flags=1, scales_in=given)
    to = wl.token_offsets
    w4 = wl.pool_weights()
    for b in range(wl.batch):
        ref = oracle.pool_given_scale(db.host["keys"][to[b]: to[b + 1]], w4, float(given[b]))
        got = H.pooled_logical(db2, b)
        assert np.max(np.abs(got.astype(int) - ref.astype(int))) <= 1
        assert got.max() <= 127 and got.min() >= -127


@pytest.mark.parametrize("k", [512, 1, 13])
def test_topk_decode_parity_ragged(ragged_batch, k):
    db = ragged_batch
    H.log(f"topk decode k={k}")
    idx, cnt, sc, _ = H.run_topk(db, k=k)
    wl = db.wl

    def one(b):
        S = H.oracle_scores_for(db, b)
        G = wl.groups(b)
        assert np.array_equal(sc[b, :G].astype(np.int64), S), f"seq {b} (L={wl.lens[b]}): scores differ"
        H.check_topk_row(S, k, idx[b], int(cnt[b]))
        return True

    assert all(oracle.map_rows(one, range(wl.batch)))


def test_topk_decode_without_score_output_matches(ragged_batch):
    db = ragged_batch
    idx1, cnt1, _, _ = H.run_topk(db, with_scores=True)
    idx2, cnt2, _, _ = H.run_topk(db, with_scores=False)
    assert np.array_equal(idx1, idx2) and np.array_equal(cnt1, cnt2)


# sequences spanning several 8192-group scoring tiles, each with a ragged last tile
MULTI_TILE = [131075, 65536, 32769, 100003, 24581]


def test_decode_multi_tile_parity():
    """Scores, selection and attention where every sequence spans several
    scoring work tiles (8192 groups each) and ends in a partial tile."""
    wl = custom("multi_tile", 13, MULTI_TILE, paged_random=True)
    db = H.make_batch(wl)
    H.run_pool(db)
    H.check_pool(db)
    idx, cnt, sc, _ = H.run_topk(db, with_scores=True)
    idx2, cnt2, _, _ = H.run_topk(db, with_scores=False)
    assert np.array_equal(idx, idx2) and np.array_equal(cnt, cnt2)
    for b in range(wl.batch):
        S = H.oracle_scores_for(db, b)
        G = wl.groups(b)
        assert np.array_equal(sc[b, :G].astype(np.int64), S), f"scores of sequence {b}"
        H.check_topk_row(S, 512, idx[b], int(cnt[b]))
    out, lse = H.run_attention(db, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), 512)
    q, lat, to = db.host["q_attn"], db.host["latent"], wl.token_offsets
    for b in range(wl.batch):
        L = wl.lens[b]
        ref, ref_lse = oracle.attention(q[b], lat[to[b]: to[b + 1]], L, L - 1, idx[b], int(cnt[b]), SM_SCALE)
        H.attention_tolerance(out[b], ref, lse[b], ref_lse)


def _batch_with_keys(name, lens, keys_logical, seed=5, paged=True):
    wl = custom(name, seed, lens, paged_random=paged)
    db = H.make_batch(wl, with_keys=False, with_latent=False)
    db.host["keys"] = keys_logical
    db.keys = H.pool_from_logical(wl, keys_logical, 256, H.NAN_BF16)
    H.run_pool(db)
    return db


def test_topk_ties_from_repeated_keys():
    """Pooled rows drawn from 3 distinct rows: every score is one of 3 values, so
    thousands of candidates tie at the boundary (exercises the exact resolve
    both in LDS and from the global lists)."""
    lens = [40000, 9000, 3000]
    base = synth.normal_bf16(21, 1, (3, IDX_DIM))
    pick = synth.uniform_i8(21, 2, (sum(lens) // 4 + 4,), 0, 2).astype(np.int64)
    keys = np.repeat(base[pick], 4, axis=0)[: sum(lens)]
    db = _batch_with_keys("ties", lens, keys)
    for k in (512, 100):
        idx, cnt, sc, _ = H.run_topk(db, k=k)
        for b in range(len(lens)):
            S = H.oracle_scores_for(db, b)
            assert len(np.unique(S)) <= 3
            assert np.array_equal(sc[b, : db.wl.groups(b)].astype(np.int64), S)
            H.check_topk_row(S, k, idx[b], int(cnt[b]))


def _score_bin(s: int) -> int:
    """The selection's 11-bit monotone histogram key of a score (exact below 64,
    then 64 sub-bins per octave), to check that an input reaches a given path."""
    s = int(s)
    if s < 64:
        return s
    e = s.bit_length() - 1
    return ((e - 5) << 6) | ((s >> (e - 6)) & 63)


def test_topk_boundary_bin_refined():
    """Several hundred candidates share the boundary histogram bin, with 15
    distinct scores and dozens of exact ties among them: the boundary bin takes
    the second histogram level, and its sub-boundary is ranked on (score, id).
    Groups are copies of one key row with four channels moved by 0.02 per step
    (0..24 steps), placed at random over the sequence's scoring tiles plus a
    run of 700 at its end (more candidates in the last tile than its list head
    in LDS holds); every other key is zero.  Selected ids bit-exact against the oracle at k =
    512 and k = 100."""
    L, seed = 40000, 42
    G = L // 4
    base = synth.bf16_to_f32(synth.normal_bf16(seed, 1, (IDX_DIM,)))
    pos = np.unique(np.concatenate([synth.uniform_i64(seed, 2, (700,), 0, G - 1), np.arange(G - 700, G)]))
    steps = synth.uniform_i64(seed, 3, (len(pos),), 0, 24)
    rows = np.repeat(base[None, :], len(pos), axis=0)
    rows[:, :4] += 0.02 * steps[:, None]
    bits = _to_bf16_bits(rows)
    keys = np.zeros((L, IDX_DIM), np.uint16)
    for t in range(4):
        keys[pos * 4 + t] = bits
    db = _batch_with_keys("refine", [L], keys, seed=seed)
    res = {k: H.run_topk(db, k=k) for k in (512, 100)}
    S = H.oracle_scores_for(db, 0)
    bins = np.array([_score_bin(x) for x in S])
    for k in (512, 100):
        bstar = np.sort(bins)[::-1][k - 1]
        nb = int((bins == bstar).sum())
        assert 128 < nb <= 2048 and len(np.unique(S[bins == bstar])) > 2, "input must reach the refined boundary"
        idx, cnt, sc, _ = res[k]
        assert np.array_equal(sc[0, :G].astype(np.int64), S)
        H.check_topk_row(S, k, idx[0], int(cnt[0]))


def test_topk_all_scores_equal():
    lens = [30000, 5000]
    keys = np.zeros((sum(lens), IDX_DIM), np.uint16)
    db = _batch_with_keys("zero", lens, keys)
    idx, cnt, sc, _ = H.run_topk(db)
    assert not np.any(sc[0, :7500]) and not np.any(sc[1, :1250])
    for b in range(2):
        assert cnt[b] == 512 and np.array_equal(idx[b], np.arange(512))


def test_topk_rows_from_scores_in():
    m = H.isa()
    rng = np.random.default_rng(3)
    rows = []
    rows.append(rng.integers(0, 2**31 - 1, size=70000))
    rows.append(rng.integers(0, 50, size=70000))                   # heavy ties
    r = rng.integers(0, 10**7, size=70000); r[rng.random(70000) < 0.7] = -1
    rows.append(r)                                                  # masked entries
    r = np.full(70000, -1); r[[5, 77, 69999]] = [3, 3, 0]
    rows.append(r)                                                  # fewer than k valid
    rows.append(np.full(70000, 12345))                              # all equal, > ROW_CAND in the boundary
    r = rng.integers(0, 1000, size=70000); r[60000:] = -1
    rows.append(r)
    S = np.stack(rows).astype(np.int32)
    for k in (512, 7):
        sd = torch.from_numpy(S).cuda()
        idx = torch.full((S.shape[0], k), -7, dtype=torch.int32, device="cuda")
        cnt = torch.zeros(S.shape[0], dtype=torch.int32, device="cuda")
        ws = m.alloc_workspace(m.workspace_size(m.ISA_OP_INDEXER_TOPK, None))
        m.isa_indexer_topk(None, None, None, None, sd, S.shape[0], S.shape[1], k, idx, cnt, None, ws)
        torch.cuda.synchronize()
        idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
        for i in range(S.shape[0]):
            H.check_topk_row(S[i].astype(np.int64), k, idx[i], int(cnt[i]))


def test_attention_parity_ragged(ragged_batch):
    db = ragged_batch
    wl = db.wl
    H.log("attention ragged")
    idx, cnt, _, _ = H.run_topk(db, with_scores=False)
    out, lse = H.run_attention(db, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), 512)
    lat = db.host["latent"]
    to = wl.token_offsets
    q = db.host["q_attn"]

    def one(b):
        L = wl.lens[b]
        ref, ref_lse = oracle.attention(q[b], lat[to[b]: to[b + 1]], L, L - 1, idx[b], int(cnt[b]), SM_SCALE)
        return H.attention_tolerance(out[b], ref, lse[b], ref_lse)

    res = oracle.map_rows(one, range(wl.batch))
    H.log(f"attention worst max-abs {max(r[0] for r in res):.2e} rel {max(r[1] for r in res):.2e}")


@pytest.mark.parametrize("lens,n", [([9000, 3000, 20000, 700, 131075], 4), ([20000], 4), ([20000, 5000], 8)],
                         ids=["b5_64heads", "b1_32heads", "b2_8layers"])
def test_index_share_layers(lens, n):
    """n layers attending over one selection in one call: every layer against
    the oracle with its own query and latent cache; one layer through the
    shared call is bit-identical to the single-layer call.  Five rows make more
    than 128 (layer, row, split) units (64 heads per workgroup); one row makes
    fewer (the heads split over two workgroups); two rows take the most layers
    a call accepts (ISA_MAX_LAYERS = 8)."""
    assert n <= H.isa().ISA_MAX_LAYERS
    from synth.configs import layer_flip_view
    wl = custom("index_share", 17, lens, paged_random=True)
    db = H.make_batch(wl)
    H.run_pool(db)
    idx, cnt, _, _ = H.run_topk(db, with_scores=False)
    idx_d, cnt_d = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    pools = H.layer_latents(db, n)
    res = H.run_attention_shared(db, idx_d, cnt_d, 512, pools)
    lat, to = db.host["latent"], wl.token_offsets
    for layer in range(n):
        q = wl.q_attn(0, wl.batch, layer=layer)
        if layer:
            layer_flip_view(lat, layer).__ixor__(np.uint16(0x8000))
        try:
            for b in range(wl.batch):
                L = wl.lens[b]
                ref, ref_lse = oracle.attention(q[b], lat[to[b]: to[b + 1]], L, L - 1, idx[b], int(cnt[b]), SM_SCALE)
                H.attention_tolerance(res[layer][0][b], ref, res[layer][1][b], ref_lse)
        finally:
            if layer:
                layer_flip_view(lat, layer).__ixor__(np.uint16(0x8000))
    one = H.run_attention_shared(db, idx_d, cnt_d, 512, pools[:1])
    out1, lse1 = H.run_attention(db, idx_d, cnt_d, 512)
    assert np.array_equal(one[0][0], out1) and np.array_equal(one[0][1], lse1)


def test_append_tokens_match_repool():
    """Decode-time appends: nine tokens appended one call at a time to every
    sequence (tails of each length, group completions, page crossings), with a
    fixed scale per sequence.  After each call the group holding the new token
    matches the oracle's pooling of the extended sequence at that scale; at the
    end the key and latent pools hold the appended rows and the pooled cache is
    bit-identical to a full isa_indexpool at the same scales."""
    m = H.isa()
    L0 = np.array([1, 255, 254, 1021, 2048, 4996, 3])
    n_app = 9
    wl = custom("append", 23, list(L0 + n_app), paged_random=True)
    B, to = wl.batch, wl.token_offsets
    keys, lat = wl.keys_logical(), wl.latent_logical()
    w4 = wl.pool_weights()
    scale = np.array([oracle.pool(keys[to[b]: to[b + 1]], w4)[1] for b in range(B)], np.float32)
    scale[2] *= np.float32(0.5)  # values clamp at +-127
    # pools holding only the first L0 tokens of each sequence (NaN bits after)
    kh, lh = keys.copy(), lat.copy()
    for b in range(B):
        kh[to[b] + L0[b]: to[b + 1]] = H.NAN_BF16
        lh[to[b] + L0[b]: to[b + 1]] = H.NAN_BF16
    kd = H.pool_from_logical(wl, kh, 256, H.NAN_BF16)
    ld = H.pool_from_logical(wl, lh, 256, H.NAN_BF16)
    bt = torch.from_numpy(wl.block_table()).cuda()
    pooled = torch.zeros((wl.num_pages, 64, IDX_DIM), dtype=torch.int8, device="cuda")
    sc = torch.from_numpy(scale).cuda()
    ws = m.alloc_workspace(m.workspace_size(m.ISA_OP_INDEXPOOL, m.Seqs(list(L0 + n_app), bt, wl.num_pages)))
    m.isa_indexpool(kd, w4, m.Seqs(list(L0), bt, wl.num_pages), sc, pooled, 1, ws)
    wsa = m.alloc_workspace(m.workspace_size(m.ISA_OP_APPEND_TOKEN, None))
    for j in range(n_app):
        lens = L0 + j + 1
        seqs = m.Seqs(list(lens), bt, wl.num_pages)
        knew = torch.from_numpy(np.stack([keys[to[b] + lens[b] - 1] for b in range(B)]).view(np.int16)).cuda()
        lnew = torch.from_numpy(np.stack([lat[to[b] + lens[b] - 1] for b in range(B)]).view(np.int16)).cuda()
        m.isa_append_token(knew, lnew, w4, seqs, sc, kd, ld, pooled, wsa)
        torch.cuda.synchronize()
        for b in range(B):
            g = (lens[b] - 1) // 4
            pg = int(wl.block_table()[b, g // 64])
            got = pooled[pg, g % 64].cpu().numpy().astype(int)
            ref = oracle.pool_given_scale(keys[to[b]: to[b] + lens[b]], w4, float(scale[b]))[g].astype(int)
            assert np.max(np.abs(got - ref)) <= 1, f"sequence {b}, length {lens[b]}"
    assert m.isa_device_error(wsa) == 0
    # the appended rows landed in the key and latent pools
    btn = wl.block_table()
    for b in range(B):
        for t in range(L0[b], L0[b] + n_app):
            pg, row = int(btn[b, t // 256]), t % 256
            assert np.array_equal(kd[pg, row].cpu().numpy().view(np.uint16), keys[to[b] + t])
            assert np.array_equal(ld[pg, row].cpu().numpy().view(np.uint16), lat[to[b] + t])
    # the same cache as a full pooling of the extended sequences at the same scales
    full = torch.zeros_like(pooled)
    m.isa_indexpool(kd, w4, m.Seqs(list(L0 + n_app), bt, wl.num_pages), sc, full, 1, ws)
    torch.cuda.synchronize()
    assert m.isa_device_error(ws) == 0
    for b in range(B):
        G = (L0[b] + n_app + 3) // 4
        pages = bt[b, : (G + 63) // 64].long()
        a_ = pooled[pages].reshape(-1, IDX_DIM)[:G]
        f_ = full[pages].reshape(-1, IDX_DIM)[:G]
        assert torch.equal(a_, f_), f"sequence {b}"


@pytest.mark.parametrize("lens", [[9000, 3000, 20003, 700, 131075],
                                  [3000, 5000, 2500, 4100, 9000, 700, 3333, 6000, 2049, 4096, 8191, 12000]],
                         ids=["b5_32heads", "b12_64heads"])
def test_fp8_latent_cache(lens):
    """FP8 latent cache: every code and row scale of isa_latent_to_fp8 bit-exact
    against the oracle's quantiser (a zero row and a large outlier included), and
    attention over the FP8 cache against the oracle's attention over the same
    codes within the attention tolerance.  Five rows make at most 128 (row,
    split) units (the heads split over two workgroups), twelve make more (64
    heads per workgroup)."""
    wl = custom("fp8", 19, lens, paged_random=True)
    lat = wl.latent_logical()
    to = wl.token_offsets
    lat[to[1] + 5] = 0                                   # a zero row: scale 1, codes 0
    lat[to[2] + 77, 300] = np.uint16(0xC2C0)             # -96: a large outlier sets the row scale
    db = H.make_batch(wl, with_latent=False)
    db.host["latent"] = lat
    db.latent = H.pool_from_logical(wl, lat, 256, H.NAN_BF16)
    H.run_pool(db)
    codes, scales = H.latent_fp8(db)
    ref_c, ref_s = oracle.latent_fp8(lat)
    for b in range(wl.batch):
        t = np.arange(wl.lens[b])
        assert np.array_equal(H.logical_rows(db, codes, b, t), ref_c[to[b]: to[b + 1]]), f"codes of sequence {b}"
        assert np.array_equal(H.logical_rows(db, scales, b, t), ref_s[to[b]: to[b + 1]]), f"scales of sequence {b}"
    assert ref_s[to[1] + 5] == 1.0 and not ref_c[to[1] + 5].any()
    idx, cnt, _, _ = H.run_topk(db, with_scores=False)
    out, lse = H.run_attention_fp8(db, codes, scales, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), 512)
    q = wl.q_attn(0, wl.batch)
    for b in range(wl.batch):
        L = wl.lens[b]
        ref, ref_lse = oracle.attention_fp8(q[b], ref_c[to[b]: to[b + 1]], ref_s[to[b]: to[b + 1]], L, L - 1, idx[b],
                                            int(cnt[b]), SM_SCALE)
        # sequence 2 carries the planted -96, held to the same bound as the rest
        H.attention_tolerance(out[b], ref, lse[b], ref_lse)


def test_kda_decode_steps():
    """Linear-attention (KDA) layer: six decode steps of 96 (sequence, head)
    units on the GPU, the oracle stepping the same inputs from the same initial
    state.  Bars, from the arithmetic: the kernel computes in fp32, so after one
    step a state element may differ from the oracle's nearest bf16 by one bf16
    step plus the fp32 error of u = S'^T k; later steps start from states that
    differ by that much, and the bound carries the difference through the decay
    and the update exactly (see below).  Outputs: rel-L2 1e-4, and per element
    1e-3 plus what the entering state difference can move the read-out."""
    from synth.configs import kda_inputs, kda_state
    m = H.isa()
    n, steps, seed = 96, 6, 29
    st_host = kda_state(seed, n)
    st_ref = st_host.copy()
    st = torch.from_numpy(st_host.view(np.int16)).cuda()
    out = torch.empty((n, 128), dtype=torch.float32, device="cuda")
    ws = m.alloc_workspace(m.workspace_size(m.ISA_OP_KDA_STEP, None))
    exact = 0
    prev_bound = np.zeros((n, 128, 128))  # both sides start from the same state
    for step in range(steps):
        q, k, v, alpha, beta = kda_inputs(seed, n, step)
        dev = [torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda() for x in (q, k, v, alpha, beta)]
        m.isa_kda_decode_step(*dev, st, out, ws)
        torch.cuda.synchronize()
        refs = oracle.map_rows(lambda u: oracle.kda_step(q[u], k[u], v[u], alpha[u], float(beta[u]), st_ref[u]),
                               range(n))
        st_ref = np.stack([r[0] for r in refs])
        o_ref = np.stack([r[1] for r in refs])
        got_bits = st.cpu().numpy().view(np.uint16)
        got, ref = synth.bf16_to_f32(got_bits).astype(np.float64), synth.bf16_to_f32(st_ref).astype(np.float64)
        # a state difference B entering the step moves S'' by at most
        # alpha_i B_ij + beta |k_i| sum_l |k_l| alpha_l B_lj (through u); this
        # step's own rounding adds one bf16 step (at most 2^-7 of the value: an
        # fp32 result can land on a bf16 midpoint the exact value misses) and the
        # fp32 error of u (~1e-6 for |S| ~ 1; 1e-5 allowed)
        kf = np.abs(synth.bf16_to_f32(k).astype(np.float64))
        prop = alpha.astype(np.float64)[:, :, None] * prev_bound
        prop = prop + beta.astype(np.float64)[:, None, None] * kf[:, :, None] * np.einsum("ul,ulj->uj", kf, prop)[:, None, :]
        bound = prop + 2.0 ** -7 * np.abs(ref) + 1e-5
        assert np.all(np.abs(got - ref) <= bound), f"step {step}: state off by {np.max(np.abs(got - ref) - bound):.2e}"
        if step == 0:
            exact = np.mean(got_bits == st_ref)
        qf = np.abs(synth.bf16_to_f32(q).astype(np.float64))
        o_bound = np.einsum("ui,uij->uj", qf, prop) + 1e-3  # the read-out of the unrounded S''
        prev_bound = bound
        o = out.cpu().numpy().astype(np.float64)
        rel = np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref)
        assert rel <= 1e-4, f"step {step}: out rel-L2 {rel:.2e}"
        assert np.all(np.abs(o - o_ref) <= o_bound), f"step {step}: out off by {np.max(np.abs(o - o_ref) - o_bound):.2e}"
    assert exact > 0.999, f"only {exact:.5f} of the first step's state elements equal the oracle's bf16"
    assert m.isa_device_error(ws) == 0


def test_attention_rows_with_positions(ragged_batch):
    """Rows that map to sequences with an earlier last-visible position (prefill rows)."""
    db = ragged_batch
    wl = db.wl
    rng = np.random.default_rng(9)
    row_seq = np.array([17, 17, 17, 16, 12, 9, 0, 13, 15, 14], np.int32)
    row_pos = np.array([rng.integers(0, wl.lens[s]) for s in row_seq], np.int32)
    row_pos[0] = 0
    row_pos[1] = wl.lens[17] - 1
    rows = len(row_seq)
    # selections: random groups (sorted, unique) of each row's sequence, k=512
    k = 512
    idx = np.full((rows, k), -1, np.int32)
    cnt = np.zeros(rows, np.int32)
    for r, s in enumerate(row_seq):
        G = wl.groups(s)
        n = min(G, k if r % 2 == 0 else 37)
        idx[r, :n] = np.sort(rng.choice(G, n, replace=False))
        cnt[r] = n
    q = synth.normal_bf16(4, 6, (rows, 64, LAT_DIM))
    out, lse = H.run_attention(db, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), k, q=q,
                               row_seq=row_seq, row_pos=row_pos, rows=rows)
    lat = db.host["latent"]
    to = wl.token_offsets
    for r, s in enumerate(row_seq):
        ref, ref_lse = oracle.attention(q[r], lat[to[s]: to[s + 1]], wl.lens[s], int(row_pos[r]), idx[r],
                                        int(cnt[r]), SM_SCALE)
        H.attention_tolerance(out[r], ref, lse[r], ref_lse)


def test_prefill_scores_topk_attention():
    m = H.isa()
    L = 20003
    wl = custom("prefill_small", 31, [L], kind="prefill",
                q_pos=[0, 1, 3, 4, 5, 100, 2047, 2048, 2049, 4095, 5000, 9999, 15000, 19999, 20000, 20002] +
                list(range(18000, 18024)))
    db = H.make_batch(wl)
    H.run_pool(db)
    Q = wl.rows
    G = wl.groups(0)
    ld = (G + 3) // 4 * 4
    qh, hwh = wl.q_idx(), wl.head_w()
    qpos = wl.row_pos()
    sc = torch.full((Q, ld), -7, dtype=torch.int32, device="cuda")
    ws = m.alloc_workspace(256)
    m.isa_indexer_prefill_scores(torch.from_numpy(qh).cuda(), torch.from_numpy(hwh).cuda(),
                                 torch.from_numpy(qpos).cuda(), Q, db.pooled, db.seqs, sc, ld, ws)
    torch.cuda.synchronize()
    assert m.isa_device_error(ws) == 0
    S = sc.cpu().numpy()
    k8 = H.pooled_logical(db, 0)
    refs = oracle.map_rows(lambda i: oracle.prefill_scores(qh[i], hwh[i], int(qpos[i]), k8), range(Q))
    for i in range(Q):
        assert np.array_equal(S[i, :G].astype(np.int64), refs[i]), f"query {i} (pos {qpos[i]})"
        assert np.all(S[i, G:] == -1), "columns past the sequence must read -1 (not candidates)"
    # selection from the precomputed rows, over the whole row stride
    idx = torch.full((Q, 512), -7, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(Q, dtype=torch.int32, device="cuda")
    m.isa_indexer_topk(None, None, None, None, sc, Q, ld, 512, idx, cnt, None, ws)
    torch.cuda.synchronize()
    idxh, cnth = idx.cpu().numpy(), cnt.cpu().numpy()
    for i in range(Q):
        H.check_topk_row(refs[i], 512, idxh[i], int(cnth[i]))
    out, lse = H.run_attention(db, idx, cnt, 512, row_seq=np.zeros(Q, np.int32), row_pos=qpos, rows=Q)
    q = db.host["q_attn"]
    lat = db.host["latent"]
    for i in range(Q):
        ref, ref_lse = oracle.attention(q[i], lat, L, int(qpos[i]), idxh[i], int(cnth[i]), SM_SCALE)
        H.attention_tolerance(out[i], ref, lse[i], ref_lse)


@pytest.mark.parametrize("L,qpos", [(77, [0, 3, 4, 40, 76]), (130, [129, 64, 1])], ids=["L77", "L130"])
def test_prefill_scores_short_sequence(L, qpos):
    """Prefill scores of a sequence shorter than one 32-group key block, or
    just over it: the blocks past the range are fetched and discarded, and the
    last query pair is finished after the block loop."""
    m = H.isa()
    wl = custom("prefill_short", 37, [L], kind="prefill", q_pos=qpos)
    db = H.make_batch(wl, with_latent=False)
    H.run_pool(db)
    Q, G = wl.rows, wl.groups(0)
    qh, hwh = wl.q_idx(), wl.head_w()
    sc = torch.full((Q, G + 4), -7, dtype=torch.int32, device="cuda")
    ws = m.alloc_workspace(256)
    m.isa_indexer_prefill_scores(torch.from_numpy(qh).cuda(), torch.from_numpy(hwh).cuda(),
                                 torch.from_numpy(wl.row_pos()).cuda(), Q, db.pooled, db.seqs, sc, G + 4, ws)
    torch.cuda.synchronize()
    assert m.isa_device_error(ws) == 0
    S = sc.cpu().numpy()
    k8 = H.pooled_logical(db, 0)
    for i in range(Q):
        ref = oracle.prefill_scores(qh[i], hwh[i], int(qpos[i]), k8)
        assert np.array_equal(S[i, :G].astype(np.int64), ref), f"query {i} (pos {qpos[i]})"
        assert np.all(S[i, G:] == -1), "columns past the sequence must read -1"


def test_paging_is_invisible():
    """The same logical data at two physical placements gives bit-identical outputs."""
    lens = [9000, 3001, 20000]
    outs = []
    for paged in (False, True):
        wl = custom("perm", 13, lens, paged_random=paged)
        db = H.make_batch(wl)
        H.run_pool(db)
        idx, cnt, sc, _ = H.run_topk(db)
        out, lse = H.run_attention(db, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), 512)
        outs.append((np.concatenate([H.pooled_logical(db, b).ravel() for b in range(3)]), idx, cnt, sc, out, lse))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_repeat_runs_are_bitwise_identical(ragged_batch):
    db = ragged_batch
    r1 = H.run_topk(db)
    r2 = H.run_topk(db)
    for a, b in zip(r1[:3], r2[:3]):
        assert np.array_equal(a, b)
    i, c = torch.from_numpy(r1[0]).cuda(), torch.from_numpy(r1[1]).cuda()
    o1 = H.run_attention(db, i, c, 512)
    o2 = H.run_attention(db, i, c, 512)
    assert np.array_equal(o1[0], o2[0]) and np.array_equal(o1[1], o2[1])


def test_device_errors_are_reported_not_faulted():
    """A block table entry outside the pool and a head weight outside [0,64] set
    error bits; the kernels skip the bad accesses."""
    m = H.isa()
    wl = custom("err", 17, [3000, 700])
    db = H.make_batch(wl, with_latent=False)
    H.run_pool(db)
    bad_bt = db.bt.clone()
    bad_bt[0, 3] = wl.num_pages + 5
    seqs = m.Seqs(wl.lens, bad_bt, wl.num_pages)
    hw = wl.head_w()
    hw[0, 0] = 65  # sequence 0 is scored (sequence 1 takes the dense fallback and reads no weights)
    idx = torch.zeros((2, 512), dtype=torch.int32, device="cuda")
    cnt = torch.zeros(2, dtype=torch.int32, device="cuda")
    ws = m.alloc_workspace(m.workspace_size(m.ISA_OP_INDEXER_TOPK, seqs))
    m.isa_indexer_topk(torch.from_numpy(wl.q_idx()).cuda(), torch.from_numpy(hw).cuda(), db.pooled, seqs, None, 2,
                       0, 512, idx, cnt, None, ws)
    torch.cuda.synchronize()
    err = m.isa_device_error(ws, clear=True)
    assert err & m.DERR_PAGE_OOB and err & m.DERR_HEADW_RANGE
    assert m.isa_device_error(ws) == 0
