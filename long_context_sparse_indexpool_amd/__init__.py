"""IndexPool sparse attention on AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libisa.so`` (the HIP kernels and the C ABI of
``include/isa.h``).  Functions keep the C names; they only marshal torch tensors
(device memory and streams) into pointers, sizes and the caller's HIP stream.
Every step of the path runs in the library's kernels; there is no fallback: if
the library is not built, importing the binding raises.

Build the library with ``python long_context_sparse_indexpool_amd/build.py``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libisa.so")

IDX_DIM, IDX_HEADS, GROUP, ATT_HEADS, LAT_DIM = 128, 32, 4, 64, 512
PAGE_TOKENS, PAGE_GROUPS = 256, 64
MAX_BATCH, MAX_SEQ_LEN, MAX_K = 256, 1 << 22, 512

ISA_OK, ISA_ERR_INVALID_ARG, ISA_ERR_UNSUPPORTED, ISA_ERR_WORKSPACE, ISA_ERR_HIP = range(5)
ISA_OP_INDEXPOOL, ISA_OP_INDEXER_TOPK, ISA_OP_SPARSE_MLA, ISA_OP_PREFILL_SCORES, ISA_OP_APPEND_TOKEN = 1, 2, 3, 4, 5
ISA_OP_LATENT_FP8, ISA_OP_KDA_STEP = 6, 7
ISA_SCALE_DYNAMIC, ISA_SCALE_GIVEN = 0, 1
ISA_MAX_LAYERS = 8  # layers sharing one selection (isa_sparse_mla_decode_shared)
DERR_PAGE_OOB, DERR_HEADW_RANGE, DERR_SCORE_OVERFLOW, DERR_ROW_RANGE, DERR_NONFINITE = 1, 2, 4, 8, 16

ISA_TIMER_INDEXER_SCORE, ISA_TIMER_MLA_SPLIT = 1, 2

EXPORTS = ("isa_workspace_size", "isa_workspace_init", "isa_device_error", "isa_status_string", "isa_version",
           "isa_set_kernel_timer", "isa_indexpool", "isa_indexer_topk", "isa_sparse_mla_decode",
           "isa_sparse_mla_decode_shared", "isa_indexer_prefill_scores", "isa_append_token", "isa_latent_to_fp8",
           "isa_sparse_mla_decode_fp8", "isa_kda_decode_step", "isa_indexer_topk_noalloc",
           "isa_read_probe")
NOALLOC_TOPK_BYTES = 256 + 384 * (8 + 8192 + 68096)


class IsaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")
        self.status = status


class isa_seqs(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("max_pages", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("seq_lens_host", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run: python long_context_sparse_indexpool_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_uint32
    sp = ctypes.POINTER(isa_seqs)
    lib.isa_workspace_size.argtypes = [ctypes.c_int, sp, i32, i32]
    lib.isa_workspace_size.restype = sz
    lib.isa_workspace_init.argtypes = [vp, sz, vp]
    lib.isa_device_error.argtypes = [vp, vp, ctypes.POINTER(u32), ctypes.c_int]
    lib.isa_status_string.argtypes = [ctypes.c_int]
    lib.isa_status_string.restype = ctypes.c_char_p
    lib.isa_version.restype = ctypes.c_char_p
    lib.isa_set_kernel_timer.argtypes = [i32, vp, vp, i32]
    lib.isa_indexpool.argtypes = [vp, vp, sp, vp, vp, u32, vp, sz, vp]
    lib.isa_indexer_topk.argtypes = [vp, vp, vp, sp, vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.isa_indexer_topk_noalloc.argtypes = [vp, vp, vp, sp, i32, vp, vp, vp, i32, vp, vp]
    lib.isa_read_probe.argtypes = [vp, sz, vp, vp, vp]
    lib.isa_sparse_mla_decode.argtypes = [vp, vp, sp, vp, vp, i32, vp, vp, i32, ctypes.c_float, vp, vp, vp, sz, vp]
    lib.isa_sparse_mla_decode_shared.argtypes = [i32, vp, vp, sp, vp, vp, i32, vp, vp, i32, ctypes.c_float, vp, vp,
                                                 vp, sz, vp]
    lib.isa_indexer_prefill_scores.argtypes = [vp, vp, vp, i32, vp, sp, vp, i32, vp, sz, vp]
    lib.isa_append_token.argtypes = [vp, vp, vp, sp, vp, vp, vp, vp, vp, sz, vp]
    lib.isa_latent_to_fp8.argtypes = [vp, sp, vp, vp, vp, sz, vp]
    lib.isa_kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    lib.isa_sparse_mla_decode_fp8.argtypes = [vp, vp, vp, sp, vp, vp, i32, vp, vp, i32, ctypes.c_float, vp, vp, vp,
                                              sz, vp]
    for f in ("isa_workspace_init", "isa_device_error", "isa_set_kernel_timer", "isa_indexpool", "isa_indexer_topk",
              "isa_sparse_mla_decode", "isa_sparse_mla_decode_shared", "isa_indexer_prefill_scores",
              "isa_append_token", "isa_latent_to_fp8", "isa_sparse_mla_decode_fp8", "isa_kda_decode_step",
              "isa_indexer_topk_noalloc", "isa_read_probe"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.isa_status_string(status).decode()


def version() -> str:
    return lib.isa_version().decode()


def _check(fn: str, status: int) -> None:
    if status != ISA_OK:
        raise IsaError(fn, status)


def _stream(stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t: Optional[torch.Tensor], dtype: torch.dtype, name: str) -> Optional[int]:
    if t is None:
        return None
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    return t.data_ptr()


@dataclass
class Seqs:
    """A batch of sequences sharing page pools (marshalled into ``isa_seqs``)."""
    lens: Sequence[int]
    block_table: torch.Tensor  # int32 [B, max_pages] on the device
    num_pages: int

    def __post_init__(self):
        self._lens = (ctypes.c_int32 * len(self.lens))(*[int(x) for x in self.lens])
        bt = self.block_table
        self._c = isa_seqs(len(self.lens), bt.shape[1] if bt.dim() == 2 else 0, int(self.num_pages), 0,
                           ctypes.cast(self._lens, ctypes.c_void_p), _ptr(bt, torch.int32, "block_table"))

    @property
    def c(self) -> ctypes.POINTER(isa_seqs):
        return ctypes.byref(self._c)


def workspace_size(op: int, seqs: Optional[Seqs], rows: int = 0, cols: int = 0) -> int:
    return int(lib.isa_workspace_size(op, seqs.c if seqs is not None else None, rows, cols))


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace (zero fill is the only initialisation the library needs)."""
    return torch.zeros(max(256, (nbytes + 255) // 256 * 256), dtype=torch.uint8, device=device)


def isa_set_kernel_timer(kernel: int, starts: Sequence[torch.cuda.Event], stops: Sequence[torch.cuda.Event]) -> None:
    """Record starts[i % n] / stops[i % n] around the i-th later launch of
    ``kernel`` (ISA_TIMER_*), on the stream of the call; empty lists switch it
    off.  The events (timing-enabled, already recorded once so that they exist)
    must stay alive while the hook is set."""
    n = len(starts)
    if n != len(stops):
        raise ValueError("starts and stops differ in length")
    arr = ctypes.c_void_p * max(n, 1)
    a = arr(*[e.cuda_event for e in starts]) if n else None
    b = arr(*[e.cuda_event for e in stops]) if n else None
    _check("isa_set_kernel_timer", lib.isa_set_kernel_timer(kernel, a, b, n))


def isa_read_probe(buf: torch.Tensor, sink: torch.Tensor, clocks: Optional[torch.Tensor] = None, stream=None) -> None:
    """Read every byte of a device buffer once (HBM read-ceiling probe); sink: int32 [1];
    clocks: int64 [2] (shader cycles, 100 MHz ticks of one wave) or None."""
    _check("isa_read_probe", lib.isa_read_probe(_ptr(buf, buf.dtype, "buf"), buf.numel() * buf.element_size(),
                                                _ptr(sink, torch.int32, "sink"), _ptr(clocks, torch.int64, "clocks"),
                                                _stream(stream)))


def isa_workspace_init(ws: torch.Tensor, stream=None) -> None:
    _check("isa_workspace_init", lib.isa_workspace_init(_ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))


def isa_device_error(ws: torch.Tensor, clear: bool = False, stream=None) -> int:
    word = ctypes.c_uint32(0)
    _check("isa_device_error", lib.isa_device_error(_ptr(ws, torch.uint8, "ws"), _stream(stream),
                                                    ctypes.byref(word), int(clear)))
    return int(word.value)


def isa_indexpool(keys: torch.Tensor, w4: Sequence[float], seqs: Seqs, scales: torch.Tensor,
                  pooled: torch.Tensor, flags: int, ws: torch.Tensor, stream=None) -> None:
    """IndexPool + int8 quantisation.  keys: bf16 bits (int16/uint16 view) [pages,256,128];
    pooled: int8 [pages,64,128]; scales: fp32 [B]."""
    w = (ctypes.c_float * 4)(*[float(x) for x in w4])
    k = keys if keys.dtype == torch.int16 else keys.view(torch.int16)
    _check("isa_indexpool", lib.isa_indexpool(_ptr(k, torch.int16, "keys"), ctypes.cast(w, ctypes.c_void_p), seqs.c,
                                              _ptr(scales, torch.float32, "scales"), _ptr(pooled, torch.int8, "pooled"),
                                              flags, _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))


def isa_append_token(key_new: torch.Tensor, latent_new: Optional[torch.Tensor], w4: Sequence[float], seqs: Seqs,
                     scales: torch.Tensor, keys: torch.Tensor, latent: Optional[torch.Tensor], pooled: torch.Tensor,
                     ws: torch.Tensor, stream=None) -> None:
    """Append one token per sequence (seqs holds the lengths after the append):
    key_new bf16 bits [B,128], latent_new bf16 bits [B,512] or None."""
    w = (ctypes.c_float * 4)(*[float(x) for x in w4])
    v16 = lambda t: None if t is None else (t if t.dtype == torch.int16 else t.view(torch.int16))
    _check("isa_append_token", lib.isa_append_token(
        _ptr(v16(key_new), torch.int16, "key_new"), _ptr(v16(latent_new), torch.int16, "latent_new"),
        ctypes.cast(w, ctypes.c_void_p), seqs.c, _ptr(scales, torch.float32, "scales"),
        _ptr(v16(keys), torch.int16, "keys"), _ptr(v16(latent), torch.int16, "latent"),
        _ptr(pooled, torch.int8, "pooled"), _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))


def isa_latent_to_fp8(latent: torch.Tensor, seqs: Seqs, codes: torch.Tensor, row_scales: torch.Tensor,
                      ws: torch.Tensor, stream=None) -> None:
    """bf16 latent pool [pages,256,512] -> E4M3 codes uint8 [pages,256,512] and fp32 row scales [pages,256]."""
    lat = latent if latent.dtype == torch.int16 else latent.view(torch.int16)
    _check("isa_latent_to_fp8", lib.isa_latent_to_fp8(
        _ptr(lat, torch.int16, "latent"), seqs.c, _ptr(codes, torch.uint8, "codes"),
        _ptr(row_scales, torch.float32, "row_scales"), _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))


def isa_sparse_mla_decode_fp8(q: torch.Tensor, codes: torch.Tensor, row_scales: torch.Tensor, seqs: Seqs,
                              row_seq: Optional[torch.Tensor], row_pos: Optional[torch.Tensor], rows: int,
                              idx: torch.Tensor, count: torch.Tensor, k: int, sm_scale: float, out: torch.Tensor,
                              lse: Optional[torch.Tensor], ws: torch.Tensor, stream=None) -> None:
    qq = q if q.dtype == torch.int16 else q.view(torch.int16)
    _check("isa_sparse_mla_decode_fp8", lib.isa_sparse_mla_decode_fp8(
        _ptr(qq, torch.int16, "q"), _ptr(codes, torch.uint8, "codes"), _ptr(row_scales, torch.float32, "row_scales"),
        seqs.c, _ptr(row_seq, torch.int32, "row_seq"), _ptr(row_pos, torch.int32, "row_pos"), rows,
        _ptr(idx, torch.int32, "idx"), _ptr(count, torch.int32, "count"), k, float(sm_scale),
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"), _ptr(ws, torch.uint8, "ws"), ws.numel(),
        _stream(stream)))


def isa_kda_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
                        state: torch.Tensor, out: torch.Tensor, ws: torch.Tensor, stream=None) -> None:
    """One KDA decode step for n units: q, k, v bf16 bits [n,128]; alpha fp32 [n,128];
    beta fp32 [n]; state bf16 bits [n,128,128] (in place); out fp32 [n,128]."""
    v16 = lambda t: t if t.dtype == torch.int16 else t.view(torch.int16)
    n = int(beta.numel())
    _check("isa_kda_decode_step", lib.isa_kda_decode_step(
        _ptr(v16(q), torch.int16, "q"), _ptr(v16(k), torch.int16, "k"), _ptr(v16(v), torch.int16, "v"),
        _ptr(alpha, torch.float32, "alpha"), _ptr(beta, torch.float32, "beta"), _ptr(v16(state), torch.int16, "state"),
        _ptr(out, torch.float32, "out"), n, _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))


def isa_indexer_topk(q: Optional[torch.Tensor], head_w: Optional[torch.Tensor], pooled: Optional[torch.Tensor],
                     seqs: Optional[Seqs], scores_in: Optional[torch.Tensor], rows: int, ld_scores: int, k: int,
                     out_idx: torch.Tensor, out_count: torch.Tensor, scores_out: Optional[torch.Tensor],
                     ws: torch.Tensor, stream=None) -> None:
    _check("isa_indexer_topk", lib.isa_indexer_topk(
        _ptr(q, torch.int8, "q"), _ptr(head_w, torch.int8, "head_w"), _ptr(pooled, torch.int8, "pooled"),
        seqs.c if seqs is not None else None, _ptr(scores_in, torch.int32, "scores_in"), rows, ld_scores, k,
        _ptr(out_idx, torch.int32, "out_idx"), _ptr(out_count, torch.int32, "out_count"),
        _ptr(scores_out, torch.int32, "scores_out"), _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))


def isa_indexer_topk_noalloc(q: torch.Tensor, head_w: torch.Tensor, pooled: torch.Tensor, seqs: Seqs, k: int,
                             out_idx: torch.Tensor, out_count: torch.Tensor, scores_out: Optional[torch.Tensor],
                             ld_scores: int, err_word: torch.Tensor, stream=None) -> None:
    """Decode-mode top-k on the library's own device scratch (no workspace);
    err_word: int32 [1] device tensor receiving the device error bits."""
    _check("isa_indexer_topk_noalloc", lib.isa_indexer_topk_noalloc(
        _ptr(q, torch.int8, "q"), _ptr(head_w, torch.int8, "head_w"), _ptr(pooled, torch.int8, "pooled"), seqs.c, k,
        _ptr(out_idx, torch.int32, "out_idx"), _ptr(out_count, torch.int32, "out_count"),
        _ptr(scores_out, torch.int32, "scores_out"), ld_scores, _ptr(err_word, torch.int32, "err_word"),
        _stream(stream)))


def isa_sparse_mla_decode(q: torch.Tensor, latent: torch.Tensor, seqs: Seqs, row_seq: Optional[torch.Tensor],
                          row_pos: Optional[torch.Tensor], rows: int, idx: torch.Tensor, count: torch.Tensor, k: int,
                          sm_scale: float, out: torch.Tensor, lse: Optional[torch.Tensor], ws: torch.Tensor,
                          stream=None) -> None:
    qq = q if q.dtype == torch.int16 else q.view(torch.int16)
    lat = latent if latent.dtype == torch.int16 else latent.view(torch.int16)
    _check("isa_sparse_mla_decode", lib.isa_sparse_mla_decode(
        _ptr(qq, torch.int16, "q"), _ptr(lat, torch.int16, "latent"), seqs.c, _ptr(row_seq, torch.int32, "row_seq"),
        _ptr(row_pos, torch.int32, "row_pos"), rows, _ptr(idx, torch.int32, "idx"),
        _ptr(count, torch.int32, "count"), k, float(sm_scale), _ptr(out, torch.float32, "out"),
        _ptr(lse, torch.float32, "lse"), _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))


def isa_sparse_mla_decode_shared(q: Sequence[torch.Tensor], latent: Sequence[torch.Tensor], seqs: Seqs,
                                 row_seq: Optional[torch.Tensor], row_pos: Optional[torch.Tensor], rows: int,
                                 idx: torch.Tensor, count: torch.Tensor, k: int, sm_scale: float,
                                 out: Sequence[torch.Tensor], lse: Optional[Sequence[torch.Tensor]], ws: torch.Tensor,
                                 stream=None) -> None:
    """Attention of len(q) layers that reuse one selection: lists of per-layer
    tensors, laid out as the arguments of isa_sparse_mla_decode."""
    n = len(q)
    if len(latent) != n or len(out) != n or (lse is not None and len(lse) != n):
        raise ValueError("q, latent, out (and lse) need one tensor per layer")
    arr = ctypes.c_void_p * max(n, 1)
    qs = arr(*[_ptr(t if t.dtype == torch.int16 else t.view(torch.int16), torch.int16, "q") for t in q])
    ls = arr(*[_ptr(t if t.dtype == torch.int16 else t.view(torch.int16), torch.int16, "latent") for t in latent])
    os_ = arr(*[_ptr(t, torch.float32, "out") for t in out])
    lses = arr(*[_ptr(t, torch.float32, "lse") for t in lse]) if lse is not None else None
    _check("isa_sparse_mla_decode_shared", lib.isa_sparse_mla_decode_shared(
        n, ctypes.cast(qs, ctypes.c_void_p), ctypes.cast(ls, ctypes.c_void_p), seqs.c,
        _ptr(row_seq, torch.int32, "row_seq"), _ptr(row_pos, torch.int32, "row_pos"), rows,
        _ptr(idx, torch.int32, "idx"), _ptr(count, torch.int32, "count"), k, float(sm_scale),
        ctypes.cast(os_, ctypes.c_void_p), ctypes.cast(lses, ctypes.c_void_p) if lses is not None else None,
        _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))


def isa_indexer_prefill_scores(q: torch.Tensor, head_w: torch.Tensor, q_pos: torch.Tensor, Q: int,
                               pooled: torch.Tensor, seqs: Seqs, scores: torch.Tensor, ld_scores: int,
                               ws: torch.Tensor, stream=None) -> None:
    _check("isa_indexer_prefill_scores", lib.isa_indexer_prefill_scores(
        _ptr(q, torch.int8, "q"), _ptr(head_w, torch.int8, "head_w"), _ptr(q_pos, torch.int32, "q_pos"), Q,
        _ptr(pooled, torch.int8, "pooled"), seqs.c, _ptr(scores, torch.int32, "scores"), ld_scores,
        _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))
