"""The seeded input generator: determinism, chunk independence, ranges, rounding."""
import numpy as np

import synth
import synth.configs as cfgs


def test_counter_based_chunks_are_independent():
    a = synth.normal_bf16(3, 5, (3 << 20,))
    b = synth.normal_bf16(3, 5, (1000,), start=(2 << 20) + 17)
    assert np.array_equal(a[(2 << 20) + 17:(2 << 20) + 1017], b)
    assert np.array_equal(a, synth.normal_bf16(3, 5, (3 << 20,)))
    assert not np.array_equal(a[:1000], synth.normal_bf16(4, 5, (1000,)))
    assert not np.array_equal(a[:1000], synth.normal_bf16(3, 6, (1000,)))


def test_normal_moments_and_bf16_rounding():
    x64 = synth.normal_f64(11, 1, (1 << 20,))
    assert abs(x64.mean()) < 5e-3 and abs(x64.std() - 1) < 5e-3
    bits = synth.normal_bf16(11, 1, (1 << 20,))
    xb = synth.bf16_to_f32(bits).astype(np.float64)
    # round to nearest: error at most half a bf16 ulp of the value
    ulp = np.ldexp(1.0, np.floor(np.log2(np.abs(x64))).astype(int) - 7)
    assert np.all(np.abs(xb - x64) <= ulp / 2 * (1 + 1e-12))


def test_uniform_int_ranges():
    q = synth.uniform_i8(0, 3, (200000,), -127, 127)
    assert q.min() == -127 and q.max() == 127
    w = synth.uniform_i8(0, 4, (200000,), 0, 64)
    assert w.min() == 0 and w.max() == 64
    counts = np.bincount(w, minlength=65)
    assert counts.min() > 0.8 * 200000 / 65


def test_workload_shapes():
    w = cfgs.workload(4)
    assert w.batch == 32
    assert all(512 <= L < (1 << 20) for L in w.lens)
    bt = w.block_table()
    assert bt.shape == (32, w.max_pages)
    used = bt[bt >= 0]
    assert len(used) == w.num_pages and len(np.unique(used)) == w.num_pages
    assert not w.is_identity_dense()
    assert cfgs.workload(2).is_identity_dense()
    w3 = cfgs.workload(3)
    assert w3.rows == 2048 and w3.row_pos()[0] == 1046528 and w3.row_pos()[-1] == 1048575
    p = cfgs.workload(0).pool_weights()
    assert p.dtype == np.float32 and abs(float(p.astype(np.float64).sum()) - 1) < 1e-6


def test_scatter_pages_roundtrip():
    w = cfgs.custom("t", 9, [300, 5, 777], paged_random=True)
    lat = w.latent_logical()
    pool = w.scatter_pages(lat, 256, 0xFFFF)
    bt = w.block_table()
    to = w.token_offsets
    for b, L in enumerate(w.lens):
        for t in (0, L // 2, L - 1):
            assert np.array_equal(pool[bt[b, t // 256], t % 256], lat[to[b] + t])
