"""The C ABI on the CPU: the library loads, exports every function include/isa.h
declares, and rejects invalid arguments synchronously, before any HIP call
(so these run without a GPU).  No compute call is made here."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "isa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(isa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def m():
    import long_context_sparse_indexpool_amd as pkg
    return pkg


def test_header_declares_the_four_calls():
    names = declared_functions()
    for f in ("isa_indexpool", "isa_indexer_topk", "isa_sparse_mla_decode", "isa_indexer_prefill_scores"):
        assert f in names


def test_every_declared_symbol_is_exported(m):
    lib = ctypes.CDLL(m.LIB_PATH)
    missing = [f for f in declared_functions() if not hasattr(lib, f)]
    assert not missing, missing
    assert set(declared_functions()) == set(m.EXPORTS)


def test_version_and_status_strings(m):
    assert "gfx950" in m.version()
    assert m.status_string(m.ISA_OK) == "ok"
    assert "workspace" in m.status_string(m.ISA_ERR_WORKSPACE)


class FakeSeqs:
    """An isa_seqs with host lengths and a fake (never dereferenced) block table."""

    def __init__(self, m, lens, max_pages=None, num_pages=1000, bt_ptr=0x10000, reserved=0):
        self.lens = (ctypes.c_int32 * len(lens))(*lens)
        mp = max_pages if max_pages is not None else max(1, max((L + 255) // 256 for L in lens))
        self.s = m.isa_seqs(len(lens), mp, num_pages, reserved, ctypes.cast(self.lens, ctypes.c_void_p), bt_ptr)

    @property
    def c(self):
        return ctypes.byref(self.s)


P = 0x100000  # fake, 16-byte aligned device address (never dereferenced: validation fails first)


def test_workspace_sizes(m):
    s = FakeSeqs(m, [8192])
    assert m.lib.isa_workspace_size(m.ISA_OP_INDEXPOOL, s.c, 0, 0) % 256 == 0
    dec = m.lib.isa_workspace_size(m.ISA_OP_INDEXER_TOPK, s.c, 1, 0)
    assert dec >= 256 + 2048 * 4 + 2048 * 8 * 1
    assert m.lib.isa_workspace_size(m.ISA_OP_INDEXER_TOPK, None, 4, 100) == 256
    assert m.lib.isa_workspace_size(m.ISA_OP_SPARSE_MLA, s.c, 2048, 0) == 256      # one split per row
    assert m.lib.isa_workspace_size(m.ISA_OP_SPARSE_MLA, s.c, 8, 0) > 256 * 1024   # split partials
    assert m.lib.isa_workspace_size(99, s.c, 1, 0) == 0
    assert m.lib.isa_workspace_size(m.ISA_OP_INDEXPOOL, FakeSeqs(m, [0]).c, 0, 0) == 0


@pytest.mark.parametrize("case", ["null_keys", "misaligned", "bad_flag", "zero_len", "too_long", "pages_short",
                                  "reserved", "batch_too_big", "ws_small"])
def test_indexpool_rejects(m, case):
    w4 = (ctypes.c_float * 4)(0.25, 0.25, 0.25, 0.25)
    keys, pooled, scales, ws, wsb, flags = P, P, P, P, 1 << 30, 0
    lens = [1000]
    kw = {}
    if case == "null_keys":
        keys = None
    elif case == "misaligned":
        pooled = P + 8
    elif case == "bad_flag":
        flags = 7
    elif case == "zero_len":
        lens = [0]
    elif case == "too_long":
        lens = [(1 << 22) + 1]
    elif case == "pages_short":
        kw["max_pages"] = 1
    elif case == "reserved":
        kw["reserved"] = 1
    elif case == "batch_too_big":
        lens = [10] * 257
    elif case == "ws_small":
        wsb = 100
    s = FakeSeqs(m, lens, **kw)
    rc = m.lib.isa_indexpool(keys, ctypes.cast(w4, ctypes.c_void_p), s.c, scales, pooled, flags, ws, wsb, None)
    assert rc == (m.ISA_ERR_WORKSPACE if case == "ws_small" else m.ISA_ERR_INVALID_ARG)


@pytest.mark.parametrize("case", ["k0", "k513", "rows_mismatch", "null_q", "ld_small", "ws_small",
                                  "scores_in_rows0", "misaligned_idx"])
def test_indexer_topk_rejects(m, case):
    s = FakeSeqs(m, [8192, 100])
    q, hw, pooled, sin, rows, ld, k, idx, cnt, sout, wsb = P, P, P, None, 2, 0, 512, P, P, None, 1 << 30
    if case == "k0":
        k = 0
    elif case == "k513":
        k = 513
    elif case == "rows_mismatch":
        rows = 3
    elif case == "null_q":
        q = None
    elif case == "ld_small":
        sout, ld = P, 100
    elif case == "ws_small":
        wsb = 1000
    elif case == "scores_in_rows0":
        sin, rows = P, 0
    elif case == "misaligned_idx":
        idx = P + 4
    rc = m.lib.isa_indexer_topk(q, hw, pooled, s.c, sin, rows, ld, k, idx, cnt, sout, P, wsb, None)
    assert rc == (m.ISA_ERR_WORKSPACE if case == "ws_small" else m.ISA_ERR_INVALID_ARG)


@pytest.mark.parametrize("case", ["null_out", "bad_scale", "rows_gt_batch", "k0", "ws_small", "nan_scale"])
def test_sparse_mla_rejects(m, case):
    s = FakeSeqs(m, [8192] * 8)
    rows, k, scale, out, wsb = 8, 512, 0.044, P, 1 << 30
    if case == "null_out":
        out = None
    elif case == "bad_scale":
        scale = 0.0
    elif case == "nan_scale":
        scale = float("nan")
    elif case == "rows_gt_batch":
        rows = 9
    elif case == "k0":
        k = 0
    elif case == "ws_small":
        wsb = 1000
    rc = m.lib.isa_sparse_mla_decode(P, P, s.c, None, None, rows, P, P, k, scale, out, None, P, wsb, None)
    assert rc == (m.ISA_ERR_WORKSPACE if case == "ws_small" else m.ISA_ERR_INVALID_ARG)


def test_shared_attention_workspace_scales_with_layers(m):
    s = FakeSeqs(m, [1 << 20] * 8)
    one = m.lib.isa_workspace_size(m.ISA_OP_SPARSE_MLA, s.c, 8, 1)
    assert m.lib.isa_workspace_size(m.ISA_OP_SPARSE_MLA, s.c, 8, 0) == one
    four = m.lib.isa_workspace_size(m.ISA_OP_SPARSE_MLA, s.c, 8, 4)
    assert four > one and four % 256 == 0
    assert m.lib.isa_workspace_size(m.ISA_OP_SPARSE_MLA, s.c, 8, m.ISA_MAX_LAYERS + 1) == 0


@pytest.mark.parametrize("case", ["layers0", "too_many", "null_array", "null_entry", "misaligned_entry",
                                  "null_lse_entry", "ws_small", "k0"])
def test_shared_attention_rejects(m, case):
    s = FakeSeqs(m, [8192] * 8)
    n, k, wsb = 4, 512, 1 << 30
    arr = ctypes.c_void_p * 8
    q, lat, out = arr(*[P] * 8), arr(*[P] * 8), arr(*[P] * 8)
    lse = None
    if case == "layers0":
        n = 0
    elif case == "too_many":
        n = m.ISA_MAX_LAYERS + 1
    elif case == "null_array":
        q = None
    elif case == "null_entry":
        lat[2] = None
    elif case == "misaligned_entry":
        out[3] = P + 8
    elif case == "null_lse_entry":
        lse = arr(*[P] * 8)
        lse[1] = None
    elif case == "ws_small":
        wsb = 1000
    elif case == "k0":
        k = 0
    c = lambda a: ctypes.cast(a, ctypes.c_void_p) if a is not None else None
    rc = m.lib.isa_sparse_mla_decode_shared(n, c(q), c(lat), s.c, None, None, 8, P, P, k, 0.044, c(out), c(lse), P,
                                            wsb, None)
    assert rc == (m.ISA_ERR_WORKSPACE if case == "ws_small" else m.ISA_ERR_INVALID_ARG)


@pytest.mark.parametrize("case", ["null_key", "latent_mismatch", "misaligned", "nan_w", "ws_small", "zero_len",
                                  "pages_short"])
def test_append_token_rejects(m, case):
    lens, mp = [257, 1024, 5], None
    key, lat_new, lat, wsb = P, P, P, 256
    w = (ctypes.c_float * 4)(0.25, 0.25, 0.25, 0.25)
    if case == "null_key":
        key = None
    elif case == "latent_mismatch":
        lat = None
    elif case == "misaligned":
        key = P + 2
    elif case == "nan_w":
        w[2] = float("nan")
    elif case == "ws_small":
        wsb = 128
    elif case == "zero_len":
        lens = [257, 0, 5]
    elif case == "pages_short":
        mp = 1  # 257 tokens need two pages
    s = FakeSeqs(m, lens, max_pages=mp)
    rc = m.lib.isa_append_token(key, lat_new, ctypes.cast(w, ctypes.c_void_p), s.c, P, P, lat, P, P, wsb, None)
    assert rc == (m.ISA_ERR_WORKSPACE if case == "ws_small" else m.ISA_ERR_INVALID_ARG)
    assert m.lib.isa_workspace_size(m.ISA_OP_APPEND_TOKEN, FakeSeqs(m, [5]).c, 0, 0) == 256


@pytest.mark.parametrize("case", ["null_codes", "misaligned_scales", "ws_small"])
def test_fp8_latent_rejects(m, case):
    s = FakeSeqs(m, [8192] * 4)
    codes, scl, wsb = P, P, 256
    if case == "null_codes":
        codes = None
    elif case == "misaligned_scales":
        scl = P + 4
    elif case == "ws_small":
        wsb = 100
    rc = m.lib.isa_latent_to_fp8(P, s.c, codes, scl, P, wsb, None)
    assert rc == (m.ISA_ERR_WORKSPACE if case == "ws_small" else m.ISA_ERR_INVALID_ARG)
    assert m.lib.isa_workspace_size(m.ISA_OP_LATENT_FP8, s.c, 0, 0) == 256


@pytest.mark.parametrize("case", ["null_scales", "misaligned_codes", "k0", "ws_small"])
def test_sparse_mla_fp8_rejects(m, case):
    s = FakeSeqs(m, [8192] * 8)
    codes, scl, k, wsb = P, P, 512, 1 << 30
    if case == "null_scales":
        scl = None
    elif case == "misaligned_codes":
        codes = P + 8
    elif case == "k0":
        k = 0
    elif case == "ws_small":
        wsb = 1000
    rc = m.lib.isa_sparse_mla_decode_fp8(P, codes, scl, s.c, None, None, 8, P, P, k, 0.044, P, None, P, wsb, None)
    assert rc == (m.ISA_ERR_WORKSPACE if case == "ws_small" else m.ISA_ERR_INVALID_ARG)


@pytest.mark.parametrize("case", ["null_state", "misaligned_alpha", "n0", "ws_small"])
def test_kda_step_rejects(m, case):
    st, al, n, wsb = P, P, 256, 256
    if case == "null_state":
        st = None
    elif case == "misaligned_alpha":
        al = P + 4
    elif case == "n0":
        n = 0
    elif case == "ws_small":
        wsb = 64
    rc = m.lib.isa_kda_decode_step(P, P, P, al, P, st, P, n, P, wsb, None)
    assert rc == (m.ISA_ERR_WORKSPACE if case == "ws_small" else m.ISA_ERR_INVALID_ARG)
    assert m.lib.isa_workspace_size(m.ISA_OP_KDA_STEP, None, 0, 0) == 256


@pytest.mark.parametrize("case", ["batch2", "q0", "ld_small", "null_pos"])
def test_prefill_scores_rejects(m, case):
    s = FakeSeqs(m, [1 << 20] if case != "batch2" else [1000, 1000])
    Q, ld, qpos = 2048, 1 << 18, P
    if case == "q0":
        Q = 0
    elif case == "ld_small":
        ld = 1000
    elif case == "null_pos":
        qpos = None
    rc = m.lib.isa_indexer_prefill_scores(P, P, qpos, Q, P, s.c, P, ld, P, 1 << 20, None)
    assert rc == m.ISA_ERR_INVALID_ARG


def test_workspace_helpers_reject(m):
    assert m.lib.isa_workspace_init(None, 1024, None) == m.ISA_ERR_INVALID_ARG
    assert m.lib.isa_workspace_init(P, 100, None) == m.ISA_ERR_INVALID_ARG
    assert m.lib.isa_device_error(None, None, None, 0) == m.ISA_ERR_INVALID_ARG


def test_kernel_timer_rejects(m):
    """The timing hook only stores handles: unknown kernels, bad counts and NULL
    handles are rejected, clearing is accepted (no event is touched here)."""
    two = (ctypes.c_void_p * 2)(P, P)
    one_null = (ctypes.c_void_p * 2)(P, None)
    assert m.lib.isa_set_kernel_timer(0, None, None, 0) == m.ISA_ERR_INVALID_ARG
    assert m.lib.isa_set_kernel_timer(3, None, None, 0) == m.ISA_ERR_INVALID_ARG
    assert m.lib.isa_set_kernel_timer(m.ISA_TIMER_INDEXER_SCORE, None, two, 2) == m.ISA_ERR_INVALID_ARG
    assert m.lib.isa_set_kernel_timer(m.ISA_TIMER_INDEXER_SCORE, two, one_null, 2) == m.ISA_ERR_INVALID_ARG
    assert m.lib.isa_set_kernel_timer(m.ISA_TIMER_MLA_SPLIT, two, two, -1) == m.ISA_ERR_INVALID_ARG
    assert m.lib.isa_set_kernel_timer(m.ISA_TIMER_MLA_SPLIT, two, two, 4097) == m.ISA_ERR_INVALID_ARG
    for k in (m.ISA_TIMER_INDEXER_SCORE, m.ISA_TIMER_MLA_SPLIT):
        assert m.lib.isa_set_kernel_timer(k, None, None, 0) == m.ISA_OK
