"""Pins of the CPU oracle to facts other than itself.

Each test ties one oracle function to what the pages fix (tests/golden/page_facts.json),
to a closed form, to a library routine on a special case, or to brute force on
small inputs.  The cases are chosen so that a plausible slip in the oracle (a
dropped term, a wrong sign, a swapped index, a transposed operand, a missing
tail rule) fails at least one of them.  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
import synth
import synth.configs

HERE = os.path.dirname(os.path.abspath(__file__))
FACTS = json.load(open(os.path.join(HERE, "golden", "page_facts.json")))
GROUP = FACTS["group_size"]["value"]
K = FACTS["group_budget"]["value"]
SCALE = 1.0 / math.sqrt(512)


def bf16_bits(x) -> np.ndarray:
    """float -> bf16 bits for values that bf16 represents exactly (test fixtures only)."""
    f = np.asarray(x, dtype=np.float32)
    bits = f.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "fixture value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


def f32(bits) -> np.ndarray:
    return synth.bf16_to_f32(np.asarray(bits, np.uint16)).astype(np.float64)


def rand_keys(rng, L, lo=-16, hi=16):
    return bf16_bits(rng.integers(lo, hi + 1, size=(L, 128)).astype(np.float32))


W_SKEW = np.array([0.5, 0.25, 0.125, 0.125], np.float32)  # exact binary fractions, sum 1
W_RAND = None


def w_rand():
    w = synth.configs.workload(0).pool_weights()
    assert abs(float(w.astype(np.float64).sum()) - 1.0) < 1e-6
    return w


# ------------------------------------------------------------------ facts
def test_page_facts_consistent():
    assert FACTS["group_budget"]["value"] * FACTS["group_size"]["value"] == FACTS["token_budget"]["value"]
    assert FACTS["indexer_heads"]["value"] == oracle.IDX_HEADS == 32
    assert FACTS["group_size"]["value"] == oracle.GROUP == 4
    assert FACTS["rope_head_dim"]["value"] == 0


# ------------------------------------------------------------------- pool
@pytest.mark.parametrize("L", list(range(1, 14)) + [255, 256, 257, 2048, 2049])
def test_pool_row_count_is_quarter(rng, L):
    """Storage falls to a quarter: ceil(L/4) pooled rows (IndexPool section)."""
    k8, scale, amax, pooled = oracle.pool(rand_keys(rng, L), W_SKEW, want_pooled=True)
    assert k8.shape == (math.ceil(L / FACTS["pool_storage_ratio"]["value"]), 128)
    assert pooled.shape == k8.shape


@pytest.mark.parametrize("w", ["skew", "rand"])
def test_pool_equal_keys_reproduce_the_key(rng, w):
    """Weights summing to 1 reproduce a key repeated 4 times."""
    w4 = W_SKEW if w == "skew" else w_rand()
    G = 37
    base = rng.standard_normal((G, 128)).astype(np.float32)
    base_bits = (base.view(np.uint32) >> 16).astype(np.uint16)  # truncate to bf16
    keys = np.repeat(base_bits, 4, axis=0)
    _, _, _, pooled = oracle.pool(keys, w4, want_pooled=True)
    want = f32(base_bits)
    tol = 1e-15 if w == "skew" else 1e-6  # fp32 weights sum to 1 within an ulp
    assert np.max(np.abs(pooled - want) / np.maximum(np.abs(want), 1e-30)) <= tol


def test_pool_impulse_response_places_each_weight(rng):
    """A unit key at slot i of a full group pools to w_i; in a tail of r tokens to
    w_i / sum_{j<r} w_j (tail renormalisation)."""
    w4 = W_SKEW
    for L in (8, 9, 10, 11):
        G = math.ceil(L / 4)
        for t in range(L):
            keys = np.zeros((L, 128), np.uint16)
            keys[t, 5] = bf16_bits(1.0)
            _, _, _, pooled = oracle.pool(keys, w4, want_pooled=True)
            g, i = divmod(t, 4)
            r = min(4, L - 4 * g)
            expect = float(w4[i]) if r == 4 else float(w4[i]) / float(w4[:r].astype(np.float64).sum())
            assert pooled[g, 5] == pytest.approx(expect, rel=1e-15)
            others = pooled.copy()
            others[g, 5] = 0.0
            assert not np.any(others), "an impulse leaked into another group or channel"
            assert pooled.shape[0] == G


def test_pool_tail_of_equal_keys_reproduces_the_key(rng):
    for r in (1, 2, 3):
        L = 12 + r
        base = bf16_bits(rng.integers(-8, 9, size=(1, 128)).astype(np.float32))
        keys = np.repeat(base, L, axis=0)
        _, _, _, pooled = oracle.pool(keys, w_rand(), want_pooled=True)
        assert np.allclose(pooled, f32(base), rtol=1e-6, atol=0)


def test_pool_is_linear(rng):
    """pool(A + B) = pool(A) + pool(B) and pool(2A) = 2 pool(A), on keys whose sums are exact in bf16."""
    L = 203
    a_f = rng.integers(-16, 17, size=(L, 128)).astype(np.float32)
    b_f = rng.integers(-16, 17, size=(L, 128)).astype(np.float32)
    w4 = w_rand()
    pa = oracle.pool(bf16_bits(a_f), w4, want_pooled=True)[3]
    pb = oracle.pool(bf16_bits(b_f), w4, want_pooled=True)[3]
    pab = oracle.pool(bf16_bits(a_f + b_f), w4, want_pooled=True)[3]
    p2a = oracle.pool(bf16_bits(2 * a_f), w4, want_pooled=True)[3]
    assert np.max(np.abs(pab - (pa + pb))) <= 1e-12
    assert np.array_equal(p2a, 2 * pa)


def test_pool_locality(rng):
    """Group g depends on tokens 4g..4g+3 only."""
    L = 64
    keys = rand_keys(rng, L)
    base = oracle.pool(keys, W_SKEW, want_pooled=True)[3]
    for t in (0, 3, 4, 30, 63):
        k2 = keys.copy()
        k2[t] = bf16_bits(np.full(128, 100.0, np.float32))
        p2 = oracle.pool(k2, W_SKEW, want_pooled=True)[3]
        changed = np.nonzero(np.any(p2 != base, axis=1))[0]
        assert changed.tolist() == [t // 4]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_quantisation_properties(seed):
    L = 1000 + 3 * seed  # includes tails
    keys = synth.normal_bf16(seed, 99, (L, 128))
    w4 = w_rand()
    k8, scale, amax, pooled = oracle.pool(keys, w4, want_pooled=True)
    assert amax == np.max(np.abs(pooled))
    assert float(scale) == pytest.approx(amax / 127.0, rel=1e-7)
    s = amax / 127.0
    # the largest magnitude maps to +-127
    arg = np.unravel_index(np.argmax(np.abs(pooled)), pooled.shape)
    assert abs(int(k8[arg])) == 127
    # rounding error at most half a step; no -128
    assert np.max(np.abs(pooled - k8.astype(np.float64) * s)) <= s / 2 * (1 + 1e-12)
    assert k8.min() >= -127
    # sign kept, zero to zero
    nz = k8 != 0
    assert np.all(np.sign(k8[nz]) == np.sign(pooled[nz]))
    keys0 = keys.copy()
    keys0[:8] = 0
    k80, _, _, p0 = oracle.pool(keys0, w4, want_pooled=True)
    assert np.all(k80[:2] == 0) and np.all(p0[:2] == 0)


def test_quantisation_round_half_even():
    """Values exactly halfway between two steps go to the even step."""
    # pooled values 0.5, 1.5, 2.5, -0.5, -2.5 and 127 steps of scale 1 -> amax 127
    vals = np.zeros((4, 128), np.float32)
    vals[:, 0] = 127.0
    vals[:, 1] = 0.5
    vals[:, 2] = 1.5
    vals[:, 3] = 2.5
    vals[:, 4] = -0.5
    vals[:, 5] = -2.5
    keys = bf16_bits(vals)
    k8, scale, amax, _ = oracle.pool(keys, W_SKEW, want_pooled=True)
    assert amax == 127.0 and float(scale) == 1.0
    assert k8[0, :6].tolist() == [127, 0, 2, 2, 0, -2]


def test_quantisation_all_zero_keys():
    k8, scale, amax, _ = oracle.pool(np.zeros((9, 128), np.uint16), W_SKEW, want_pooled=True)
    assert amax == 0.0 and float(scale) == 1.0 and not np.any(k8)


def test_pool_given_scale_matches_dynamic_and_clamps(rng):
    keys = synth.normal_bf16(7, 99, (333, 128))
    w4 = w_rand()
    k8, scale, _, pooled = oracle.pool(keys, w4, want_pooled=True)
    assert np.array_equal(oracle.pool_given_scale(keys, w4, float(scale)), k8) or \
        np.max(np.abs(oracle.pool_given_scale(keys, w4, float(scale)).astype(int) - k8)) <= 1
    small = oracle.pool_given_scale(keys, w4, float(scale) / 4)
    assert small.max() == 127 and small.min() == -127


# ----------------------------------------------------------------- scores
def _rand_q(rng):
    return rng.integers(-127, 128, size=(32, 128)).astype(np.int8)


def _rand_k(rng, G):
    return rng.integers(-127, 128, size=(G, 128)).astype(np.int8)


@pytest.mark.parametrize("h", [0, 1, 17, 31])
def test_scores_one_hot_weight_is_relu_of_gemv(rng, h):
    """w = e_h isolates ReLU(q_h . k): a plain GEMV followed by ReLU (numpy)."""
    q, k = _rand_q(rng), _rand_k(rng, 300)
    w = np.zeros(32, np.int8)
    w[h] = 1
    want = np.maximum(k.astype(np.int64) @ q[h].astype(np.int64), 0)
    assert np.array_equal(oracle.scores(q, w, k), want)
    w[h] = 64
    assert np.array_equal(oracle.scores(q, w, k), 64 * want)


def test_scores_sign_symmetry(rng):
    """S(q) + S(-q) = sum_h w_h |q_h . k| (ReLU(x) + ReLU(-x) = |x|)."""
    q, k = _rand_q(rng), _rand_k(rng, 257)
    w = rng.integers(0, 65, size=32).astype(np.int8)
    lhs = oracle.scores(q, w, k) + oracle.scores((-q.astype(np.int16)).astype(np.int8), w, k)
    rhs = np.abs(k.astype(np.int64) @ q.astype(np.int64).T) @ w.astype(np.int64)
    assert np.array_equal(lhs, rhs)


def test_scores_zero_query_and_additive_weights(rng):
    q, k = _rand_q(rng), _rand_k(rng, 99)
    assert not np.any(oracle.scores(np.zeros((32, 128), np.int8), rng.integers(0, 65, 32).astype(np.int8), k))
    w1 = rng.integers(0, 33, 32).astype(np.int8)
    w2 = rng.integers(0, 33, 32).astype(np.int8)
    s12 = oracle.scores(q, (w1 + w2).astype(np.int8), k)
    assert np.array_equal(s12, oracle.scores(q, w1, k) + oracle.scores(q, w2, k))


def test_scores_worst_case_magnitude():
    """All q = k = 127, w = 64: S = 32 * 64 * 128 * 127^2 (beyond int32, exact in int64)."""
    q = np.full((32, 128), 127, np.int8)
    k = np.full((3, 128), 127, np.int8)
    w = np.full(32, 64, np.int8)
    assert oracle.scores(q, w, k).tolist() == [32 * 64 * 128 * 127 * 127] * 3


def test_scores_heads_are_not_channels(rng):
    """A query nonzero in one head only: the score uses that head's weight, not a channel's."""
    k = _rand_k(rng, 50)
    q = np.zeros((32, 128), np.int8)
    q[5] = rng.integers(-127, 128, 128)
    w = np.zeros(32, np.int8)
    w[5] = 3
    want = 3 * np.maximum(k.astype(np.int64) @ q[5].astype(np.int64), 0)
    assert np.array_equal(oracle.scores(q, w, k), want)
    w2 = w.copy()
    w2[5] = 0
    w2[6] = 3
    assert not np.any(oracle.scores(q, w2, k))


@pytest.mark.parametrize("pos", [0, 1, 3, 4, 7, 8, 4 * 40 + 2, 4 * 49 + 3])
def test_prefill_block_causal_mask(rng, pos):
    """Group g is visible iff g <= floor(pos/4) (the query's own group included)."""
    q, k = _rand_q(rng), _rand_k(rng, 50)
    w = rng.integers(0, 65, 32).astype(np.int8)
    S = oracle.prefill_scores(q, w, pos, k)
    last = pos // 4
    assert np.all(S[last + 1:] == -1)
    assert np.array_equal(S[: last + 1], oracle.scores(q, w, k[: last + 1]))
    assert np.all(S[: last + 1] >= 0)


# ------------------------------------------------------------------- topk
def brute_force_topk(S, K):
    """Independent formulation: rank(g) = #{g' valid: S' > S or (S' == S and g' < g)}."""
    S = np.asarray(S, np.int64)
    valid = np.nonzero(S >= 0)[0]
    if len(valid) <= K:
        return valid.astype(np.int32)
    sv = S[valid]
    ranks = np.zeros(len(valid), np.int64)
    for a in range(0, len(valid), 1024):
        blk = sv[a:a + 1024, None]
        gi = valid[a:a + 1024, None]
        ranks[a:a + 1024] = np.sum((sv[None, :] > blk) | ((sv[None, :] == blk) & (valid[None, :] < gi)), axis=1)
    return valid[ranks < K].astype(np.int32)


@pytest.mark.parametrize("G,rng_hi", [(513, 10), (600, 3), (1000, 1_000_000), (2048, 50), (4099, 7),
                                      (8192, 2 ** 31 - 1), (8192, 1000)])
def test_topk_matches_rank_count_brute_force(rng, G, rng_hi):
    S = rng.integers(0, rng_hi + 1, size=G).astype(np.int64)
    idx, cnt = oracle.topk(S, K)
    want = brute_force_topk(S, K)
    assert cnt == K == len(want)
    assert np.array_equal(idx[:cnt], want)
    assert np.all(np.diff(idx[:cnt]) > 0)


def test_topk_all_equal_takes_lowest_indices():
    idx, cnt = oracle.topk(np.full(5000, 7, np.int64), K)
    assert cnt == K and np.array_equal(idx, np.arange(K))


def test_topk_descending_scores_take_first_block():
    S = np.arange(3000, 0, -1).astype(np.int64)
    idx, cnt = oracle.topk(S, K)
    assert np.array_equal(idx, np.arange(K))
    idx, cnt = oracle.topk(S[::-1].copy(), K)
    assert np.array_equal(idx, np.arange(3000 - K, 3000))


@pytest.mark.parametrize("G", [0, 1, 5, 511, 512])
def test_topk_dense_fallback_selects_all(G):
    """At most 512 groups (fewer than 2048 positions): everything is selected."""
    S = (np.arange(G) * 7919 % 13).astype(np.int64)
    idx, cnt = oracle.topk(S, K)
    assert cnt == G
    assert np.array_equal(idx[:G], np.arange(G)) and np.all(idx[G:] == -1)


def test_topk_boundary_of_dense_regime():
    """L = 2048 tokens -> 512 groups -> dense; L = 2049 -> 513 groups -> one is dropped."""
    dense = FACTS["dense_below_positions"]["value"]
    for L, expect_all in ((dense, True), (dense + 1, False)):
        G = math.ceil(L / 4)
        S = np.ones(G, np.int64)
        idx, cnt = oracle.topk(S, K)
        assert cnt == min(G, K)
        assert expect_all == (cnt == G)


def test_topk_masked_entries_never_selected(rng):
    S = rng.integers(0, 100, size=3000).astype(np.int64)
    S[rng.random(3000) < 0.6] = -1
    idx, cnt = oracle.topk(S, K)
    assert np.all(S[idx[:cnt]] >= 0)
    assert np.array_equal(idx[:cnt], brute_force_topk(S, K))
    S2 = np.full(700, -1, np.int64)
    S2[[3, 9, 600]] = 0
    idx, cnt = oracle.topk(S2, K)
    assert cnt == 3 and idx[:3].tolist() == [3, 9, 600]


def test_topk_ties_straddling_the_threshold(rng):
    """Many copies of the threshold score at scattered indices: the lowest indices win."""
    G = 4096
    S = rng.integers(0, 1000, size=G).astype(np.int64)
    S[rng.choice(G, 400, replace=False)] = 5000   # 400 sure winners
    tie = rng.choice(np.nonzero(S < 5000)[0], 300, replace=False)
    S[tie] = 4000                                   # 300 tied for the last 112 slots
    idx, cnt = oracle.topk(S, K)
    chosen_ties = np.intersect1d(idx, tie)
    assert len(chosen_ties) == K - 400
    assert np.array_equal(chosen_ties, np.sort(tie)[: K - 400])


# -------------------------------------------------------------- attention
def _rand_bf16(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def textbook_dense(q_bits, lat_bits, T):
    """softmax(q C^T * scale) C over the first T rows with scipy's softmax / logsumexp."""
    q = f32(q_bits)
    c = f32(lat_bits[:T])
    s = (q @ c.T) * SCALE
    return softmax(s, axis=1) @ c, logsumexp(s, axis=1)


@pytest.mark.parametrize("L", [1, 2, 3, 4, 5, 100, 2047, 2048])
def test_attention_dense_fallback_is_textbook_attention(rng, L):
    """Below the budget every group is selected and the result is plain dense softmax attention."""
    q = _rand_bf16(rng, (64, 512))
    lat = _rand_bf16(rng, (L, 512))
    G = math.ceil(L / 4)
    idx, cnt = oracle.topk(np.zeros(G, np.int64), K)
    out, lse = oracle.attention(q, lat, L, L - 1, idx, cnt, SCALE)
    ref, ref_lse = textbook_dense(q, lat, L)
    assert np.max(np.abs(out - ref)) < 1e-12
    assert np.max(np.abs(lse - ref_lse)) < 1e-10


def test_attention_single_token_returns_that_row(rng):
    q = _rand_bf16(rng, (64, 512))
    lat = _rand_bf16(rng, (40, 512))
    out, lse = oracle.attention(q, lat, 40, 20, np.array([5, 1], np.int32), 2, SCALE)
    # group 5 = tokens 20..23 but pos = 20 -> only token 20; group 1 = tokens 4..7
    sel_rows = [4, 5, 6, 7, 20]
    ref, ref_lse = textbook_dense(q, lat[sel_rows], 5)
    assert np.max(np.abs(out - ref)) < 1e-12
    out1, lse1 = oracle.attention(q, lat, 40, 20, np.array([5], np.int32), 1, SCALE)
    assert np.array_equal(out1, np.broadcast_to(f32(lat[20]), (64, 512)))
    assert np.allclose(lse1, f32(q) @ f32(lat[20]) * SCALE, rtol=0, atol=1e-12)


def test_attention_identical_rows_and_zero_query(rng):
    row = _rand_bf16(rng, (1, 512))
    lat = np.repeat(row, 64, axis=0)
    q = _rand_bf16(rng, (64, 512))
    out, _ = oracle.attention(q, lat, 64, 63, np.arange(16, dtype=np.int32), 16, SCALE)
    assert np.max(np.abs(out - f32(row))) < 1e-14
    lat = _rand_bf16(rng, (64, 512))
    out, lse = oracle.attention(np.zeros((64, 512), np.uint16), lat, 64, 63, np.array([2, 9, 11], np.int32), 3,
                                SCALE)
    rows = [8, 9, 10, 11, 36, 37, 38, 39, 44, 45, 46, 47]
    assert np.max(np.abs(out - f32(lat[rows]).mean(axis=0))) < 1e-14
    assert np.allclose(lse, math.log(len(rows)), atol=1e-14)


def test_attention_order_invariance_and_causality(rng):
    q = _rand_bf16(rng, (64, 512))
    lat = _rand_bf16(rng, (400, 512))
    sel = np.array([3, 50, 7, 99, 60], np.int32)
    out, lse = oracle.attention(q, lat, 400, 250, sel, 5, SCALE)
    out2, lse2 = oracle.attention(q, lat, 400, 250, sel[::-1].copy(), 5, SCALE)
    assert np.max(np.abs(out - out2)) < 1e-12
    lat2 = lat.copy()
    lat2[251:] = _rand_bf16(rng, (149, 512))          # tokens after pos never matter
    out3, _ = oracle.attention(q, lat2, 400, 250, sel, 5, SCALE)
    assert np.array_equal(out, out3)
    lat3 = lat.copy()
    lat3[200] = _rand_bf16(rng, (1, 512))             # token 200 (group 50) does
    out4, _ = oracle.attention(q, lat3, 400, 250, sel, 5, SCALE)
    assert not np.array_equal(out, out4)
    # rows past the sequence end (t >= L) are never read
    out5, _ = oracle.attention(q, lat[:398], 398, 10_000, np.array([99], np.int32), 1, SCALE)
    ref, _ = textbook_dense(q, lat[396:398], 2)
    assert np.max(np.abs(out5 - ref)) < 1e-12


def test_attention_probabilities_sum_to_one(rng):
    """Softmax rows sum to 1: with latent rows all equal to c plus a one-hot bump the
    output's bump coordinate equals the probability mass on the bumped token."""
    q = _rand_bf16(rng, (64, 512))
    lat = np.zeros((32, 512), np.uint16)
    lat[:, 0] = bf16_bits(1.0)
    out, _ = oracle.attention(q, lat, 32, 31, np.arange(8, dtype=np.int32), 8, SCALE)
    assert np.allclose(out[:, 0], 1.0, atol=1e-15)


def test_attention_empty_selection():
    out, lse = oracle.attention(np.zeros((64, 512), np.uint16), np.zeros((8, 512), np.uint16), 8, 7,
                                np.array([-1], np.int32), 0, SCALE)
    assert not np.any(out) and np.all(np.isneginf(lse))


# ---------------------------------------------------------------------- FP8 latent cache
# OCP E4M3 facts: bias 7, 3 mantissa bits, subnormals m/8 * 2^-6, S.1111.111 = NaN,
# no infinities, so the largest finite value is 1.75 * 2^8 = 448.

def test_fp8_decode_table():
    assert oracle.fp8_decode(0x00) == 0.0 and math.copysign(1.0, oracle.fp8_decode(0x80)) == -1.0
    assert oracle.fp8_decode(0x01) == 2.0 ** -9 and oracle.fp8_decode(0x07) == 7 * 2.0 ** -9
    assert oracle.fp8_decode(0x08) == 2.0 ** -6 and oracle.fp8_decode(0x38) == 1.0
    assert oracle.fp8_decode(0x39) == 1.125 and oracle.fp8_decode(0x40) == 2.0
    assert oracle.fp8_decode(0x7E) == 448.0 and oracle.fp8_decode(0xFE) == -448.0
    assert math.isnan(oracle.fp8_decode(0x7F)) and math.isnan(oracle.fp8_decode(0xFF))
    pos = [oracle.fp8_decode(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:]))  # strictly increasing codes 0x00..0x7E
    for c in range(0x7F):
        assert oracle.fp8_decode(c | 0x80) == -pos[c]


def test_fp8_encode_round_trip_and_nearest():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.fp8_encode(oracle.fp8_decode(c)) == c
    pos = [oracle.fp8_decode(c) for c in range(0x7F)]
    for c in range(0x7E):
        lo, hi = pos[c], pos[c + 1]
        mid = (lo + hi) / 2  # exact in fp32 for these values
        assert oracle.fp8_encode(mid) == (c if c % 2 == 0 else c + 1), hex(c)  # ties to the even mantissa
        gap = hi - lo
        assert oracle.fp8_encode(lo + 0.25 * gap) == c and oracle.fp8_encode(hi - 0.25 * gap) == c + 1
        assert oracle.fp8_encode(-(lo + 0.25 * gap)) == (c | 0x80 if c else 0x80)


def test_fp8_encode_overflow_is_nan():
    assert oracle.fp8_encode(448.0) == 0x7E and oracle.fp8_encode(464.0) == 0x7E
    assert oracle.fp8_encode(464.5) == 0x7F and oracle.fp8_encode(-1e9) == 0xFF
    assert oracle.fp8_encode(float("nan")) == 0x7F


def test_latent_fp8_rows(rng):
    lat = synth.normal_bf16(31, 5, (40, 512))
    lat[3] = 0  # a zero row
    lat[5, 17] = bf16_bits([-96.0])[0]  # a row whose amax is a negative outlier
    codes, scales = oracle.latent_fp8(lat)
    x = f32(lat)
    for t in range(40):
        amax = np.float32(np.max(np.abs(x[t])))
        if amax == 0:
            assert scales[t] == 1.0 and not np.any(codes[t])
            continue
        assert scales[t] == np.float32(amax / np.float32(448.0))
        j = int(np.argmax(np.abs(x[t])))
        assert codes[t, j] == (0x7E if x[t, j] > 0 else 0xFE)  # the amax element maps to +-448
        v = np.array([oracle.fp8_decode(c) for c in codes[t]])
        y = (x[t].astype(np.float32) / scales[t]).astype(np.float64)
        # within half a spacing of the nearest code (spacing 2^(e-3), at least 2^-9)
        e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6)))
        assert np.all(np.abs(y - v) <= 2.0 ** (e - 3) / 2 + 1e-12)
        assert np.all(np.sign(v) * np.sign(y) >= 0)


def test_attention_fp8_equals_bf16_attention_on_exact_values(rng):
    """Codes with power-of-two row scales are exact bf16 values, so the FP8 cache
    and the bf16 cache of the same values must give identical attention."""
    L = 300
    codes = rng.integers(0, 0x7F, size=(L, 512)).astype(np.uint8)
    codes[codes == 0x7F] = 0x7E
    codes |= (rng.integers(0, 2, size=(L, 512)) * 0x80).astype(np.uint8)
    scales = (2.0 ** rng.integers(-6, 3, size=L)).astype(np.float32)
    vals = np.array([[oracle.fp8_decode(c) for c in row] for row in codes]) * scales[:, None]
    lat = bf16_bits(vals.astype(np.float32))
    q = synth.normal_bf16(32, 6, (64, 512))
    sel = np.sort(rng.choice(L // 4, size=40, replace=False)).astype(np.int32)
    a = oracle.attention(q, lat, L, L - 1, sel, len(sel), SCALE)
    b = oracle.attention_fp8(q, codes, scales, L, L - 1, sel, len(sel), SCALE)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = oracle.attention_fp8(q, codes, scales * np.float32(2.0), L, L - 1, sel, len(sel), SCALE)
    assert not np.allclose(c[0], a[0])  # the row scales enter the result


# ---------------------------------------------------------------------- KDA decode step
def _kda_inputs(rng, unit_k=True):
    D = 128
    q = synth.normal_bf16(41, 1, (D,))
    k = synth.normal_bf16(41, 2, (D,))
    if unit_k:
        kf = f32(k)
        k = bf16_bits((kf / np.linalg.norm(kf)).astype(np.float32).view(np.uint32).__and__(0xFFFF0000).view(np.float32))
    v = synth.normal_bf16(41, 3, (D,))
    S = synth.normal_bf16(41, 4, (D, D))
    return q, k, v, S


def _ulp_ok(got_bits, ref):
    """got (bf16 bits) is the nearest bf16 of ref: within half a bf16 spacing."""
    got = f32(got_bits)
    e = np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126)))
    return np.all(np.abs(got - ref) <= 2.0 ** (e - 8) + 1e-300)


def test_kda_no_erase_no_decay_keeps_state(rng):
    q, k, v, S = _kda_inputs(rng)
    S2, o = oracle.kda_step(q, k, v, np.ones(128, np.float32), 0.0, S)
    assert np.array_equal(S2, S)
    assert np.allclose(o, f32(S).T @ f32(q), rtol=1e-12, atol=1e-12)  # o = S^T q


def test_kda_delta_rule_is_the_pages_equation(rng):
    q, k, v, S = _kda_inputs(rng)
    for beta in (0.3, 1.0):
        S2, o = oracle.kda_step(q, k, v, np.ones(128, np.float32), beta, S)
        Sf, kf, vf = f32(S), f32(k), f32(v)
        b = float(np.float32(beta))  # the gate is an fp32 argument
        ref = Sf - b * np.outer(kf, kf @ Sf) + b * np.outer(kf, vf)
        assert _ulp_ok(S2, ref)
        assert np.allclose(o, ref.T @ f32(q), rtol=1e-10, atol=1e-10)


def test_kda_writes_the_value_at_a_unit_key(rng):
    q, k, v, S = _kda_inputs(rng)
    # a key of exactly unit norm (four channels of +-1/2) and beta = 1: the
    # delta rule replaces what the key retrieves by v, so reading the new state
    # with q = k returns v
    kb = np.zeros(128, np.float32)
    kb[[3, 17, 64, 100]] = [0.5, -0.5, 0.5, -0.5]
    k = bf16_bits(kb)
    _, o = oracle.kda_step(k, k, v, np.ones(128, np.float32), 1.0, S)
    assert np.allclose(o, f32(v), rtol=1e-12, atol=1e-12)


def test_kda_decay_scales_key_rows(rng):
    q, k, v, S = _kda_inputs(rng)
    alpha = rng.uniform(0.0, 1.0, 128).astype(np.float32)
    alpha[5] = 0.0
    S2, o = oracle.kda_step(q, k, v, alpha, 0.0, S)
    ref = alpha[:, None].astype(np.float64) * f32(S)
    assert _ulp_ok(S2, ref) and not np.any(f32(S2)[5])
    assert np.allclose(o, ref.T @ f32(q), rtol=1e-12, atol=1e-12)
