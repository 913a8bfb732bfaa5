"""CPU oracle of the IndexPool sparse-attention path (ctypes over oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the GPU library; the two meet only in the seeded inputs of ``synth``.

The C functions are reentrant and ctypes drops the GIL while they run, so the
helpers below spread independent rows (or group ranges of one row) over host
threads.  Results do not depend on the thread count: every output element is
computed by one call in a fixed order.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

IDX_DIM, IDX_HEADS, GROUP, ATT_HEADS, LAT_DIM = 128, 32, 4, 64, 512


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (no HIP headers, no GPU code)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        # ISO C mode keeps floating-point contraction off, so -O3 changes speed only
        subprocess.check_call(["gcc", "-O3", "-std=c11", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
            vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
            lib.oracle_pool.argtypes = [vp, i64, vp, vp, vp, vp, vp]
            lib.oracle_pool.restype = ctypes.c_int
            lib.oracle_pool_given_scale.argtypes = [vp, i64, vp, ctypes.c_float, vp]
            lib.oracle_pool_given_scale.restype = ctypes.c_int
            lib.oracle_scores.argtypes = [vp, vp, vp, i64, vp]
            lib.oracle_scores.restype = None
            lib.oracle_prefill_scores.argtypes = [vp, vp, i64, vp, i64, vp]
            lib.oracle_prefill_scores.restype = None
            lib.oracle_topk.argtypes = [vp, i64, i32, vp, vp]
            lib.oracle_topk.restype = ctypes.c_int
            lib.oracle_attention.argtypes = [vp, vp, i64, i64, vp, i32, ctypes.c_double, vp, vp]
            lib.oracle_attention.restype = ctypes.c_int
            lib.oracle_fp8_decode.argtypes = [ctypes.c_uint8]
            lib.oracle_fp8_decode.restype = ctypes.c_double
            lib.oracle_fp8_encode.argtypes = [ctypes.c_float]
            lib.oracle_fp8_encode.restype = ctypes.c_uint8
            lib.oracle_latent_fp8.argtypes = [vp, i64, vp, vp]
            lib.oracle_latent_fp8.restype = ctypes.c_int
            lib.oracle_attention_fp8.argtypes = [vp, vp, vp, i64, i64, vp, i32, ctypes.c_double, vp, vp]
            lib.oracle_attention_fp8.restype = ctypes.c_int
            lib.oracle_kda_step.argtypes = [vp, vp, vp, vp, ctypes.c_float, vp, vp]
            lib.oracle_kda_step.restype = ctypes.c_int
            lib.oracle_bf16_round.argtypes = [ctypes.c_double]
            lib.oracle_bf16_round.restype = ctypes.c_uint16
            _lib = lib
    return _lib


class use_library:
    """Temporarily route every wrapper through another build of oracle.c (the
    mutation tests compile deliberately broken copies on the CPU)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        _load()
        self._saved = _lib
        with _lock:
            _lib = None
        saved_path = globals()["_LIB_PATH"]
        globals()["_LIB_PATH"] = self.path
        try:
            _load()
        finally:
            globals()["_LIB_PATH"] = saved_path
        return self

    def __exit__(self, *exc):
        global _lib
        with _lock:
            _lib = self._saved
        return False


def n_threads() -> int:
    """Host threads for the oracle: every CPU in this process's affinity mask,
    capped by OMP_NUM_THREADS when the environment sets it (a machine that
    grants the process a share of its CPUs says so there)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# --------------------------------------------------------------------------- pool
def pool(keys: np.ndarray, w4: np.ndarray, want_pooled: bool = False):
    """keys: bf16 bits [L,128]. Returns (k8 [G,128] int8, scale fp32, amax, pooled or None)."""
    keys = _c(keys, np.uint16)
    w4 = _c(w4, np.float32)
    L = keys.shape[0]
    G = (L + GROUP - 1) // GROUP
    k8 = np.empty((G, IDX_DIM), np.int8)
    pooled = np.empty((G, IDX_DIM), np.float64) if want_pooled else None
    scale = ctypes.c_float()
    amax = ctypes.c_double()
    rc = _load().oracle_pool(_ptr(keys), L, _ptr(w4), _ptr(pooled) if want_pooled else None, _ptr(k8),
                             ctypes.byref(scale), ctypes.byref(amax))
    if rc != 0:
        raise ValueError(f"oracle_pool rc={rc}")
    return k8, np.float32(scale.value), amax.value, pooled


def pool_given_scale(keys: np.ndarray, w4: np.ndarray, scale: float) -> np.ndarray:
    keys = _c(keys, np.uint16)
    w4 = _c(w4, np.float32)
    L = keys.shape[0]
    k8 = np.empty(((L + GROUP - 1) // GROUP, IDX_DIM), np.int8)
    rc = _load().oracle_pool_given_scale(_ptr(keys), L, _ptr(w4), ctypes.c_float(scale), _ptr(k8))
    if rc != 0:
        raise ValueError(f"oracle_pool_given_scale rc={rc}")
    return k8


# ------------------------------------------------------------------------- scores
def scores(q: np.ndarray, w: np.ndarray, k8: np.ndarray, threads: int | None = None) -> np.ndarray:
    """q [32,128] int8, w [32] int8, k8 [G,128] int8 -> S [G] int64 (group ranges in parallel)."""
    q = _c(q, np.int8)
    w = _c(w, np.int8)
    k8 = _c(k8, np.int8)
    G = k8.shape[0]
    S = np.empty(G, np.int64)
    lib = _load()
    nt = threads or n_threads()
    per = max(4096, (G + nt - 1) // nt)
    spans = [(a, min(G, a + per)) for a in range(0, G, per)]

    def work(s):
        a, b = s
        lib.oracle_scores(_ptr(q), _ptr(w), _ptr(k8) + a * IDX_DIM, b - a, _ptr(S) + a * 8)

    if len(spans) == 1:
        work(spans[0])
    else:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(work, spans))
    return S


def prefill_scores(q: np.ndarray, w: np.ndarray, pos: int, k8: np.ndarray) -> np.ndarray:
    q = _c(q, np.int8)
    w = _c(w, np.int8)
    k8 = _c(k8, np.int8)
    G = k8.shape[0]
    S = np.empty(G, np.int64)
    _load().oracle_prefill_scores(_ptr(q), _ptr(w), int(pos), _ptr(k8), G, _ptr(S))
    return S


# --------------------------------------------------------------------------- topk
def topk(S: np.ndarray, K: int = 512):
    """S [G] (int64, valid iff >= 0) -> (idx [K] int32 ascending, -1 padded; count)."""
    S = _c(S, np.int64)
    idx = np.empty(K, np.int32)
    cnt = ctypes.c_int32()
    rc = _load().oracle_topk(_ptr(S), S.shape[0], K, _ptr(idx), ctypes.byref(cnt))
    if rc != 0:
        raise ValueError(f"oracle_topk rc={rc}")
    return idx, int(cnt.value)


# ---------------------------------------------------------------------- attention
def attention(q: np.ndarray, lat: np.ndarray, L: int, pos: int, sel: np.ndarray, count: int,
              scale: float):
    """q bf16 bits [64,512]; lat bf16 bits [>=L,512] (logical rows) -> (out [64,512] f64, lse [64] f64)."""
    q = _c(q, np.uint16)
    lat = _c(lat, np.uint16)
    sel = _c(sel, np.int32)
    out = np.empty((ATT_HEADS, LAT_DIM), np.float64)
    lse = np.empty(ATT_HEADS, np.float64)
    rc = _load().oracle_attention(_ptr(q), _ptr(lat), int(L), int(pos), _ptr(sel), int(count), float(scale),
                                  _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_attention rc={rc}")
    return out, lse


# ------------------------------------------------------------------ FP8 latent cache
def fp8_decode(code: int) -> float:
    """Value of an OCP E4M3 code (NaN for 0x7F / 0xFF)."""
    return float(_load().oracle_fp8_decode(int(code)))


def fp8_encode(x: float) -> int:
    """Nearest E4M3 code of an fp32 value (ties to even; past 464 in magnitude: NaN)."""
    return int(_load().oracle_fp8_encode(float(x)))


def latent_fp8(lat: np.ndarray):
    """bf16 bits [n,512] -> (codes uint8 [n,512], scales fp32 [n]): per-row amax/448 scale."""
    lat = _c(lat, np.uint16)
    n = lat.shape[0]
    codes = np.empty((n, LAT_DIM), np.uint8)
    scales = np.empty(n, np.float32)
    rc = _load().oracle_latent_fp8(_ptr(lat), int(n), _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError(f"oracle_latent_fp8 rc={rc}")
    return codes, scales


def attention_fp8(q: np.ndarray, codes: np.ndarray, scales: np.ndarray, L: int, pos: int, sel: np.ndarray,
                  count: int, scale: float):
    """attention() over an FP8 cache: latent value of token t = scales[t] * decode(codes[t])."""
    q = _c(q, np.uint16)
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32)
    sel = _c(sel, np.int32)
    out = np.empty((ATT_HEADS, LAT_DIM), np.float64)
    lse = np.empty(ATT_HEADS, np.float64)
    rc = _load().oracle_attention_fp8(_ptr(q), _ptr(codes), _ptr(scales), int(L), int(pos), _ptr(sel), int(count),
                                      float(scale), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_attention_fp8 rc={rc}")
    return out, lse


# ------------------------------------------------------------------ linear-attention (KDA) layers
KDA_DIM = 128


def kda_step(q: np.ndarray, k: np.ndarray, v: np.ndarray, alpha: np.ndarray, beta: float, S: np.ndarray):
    """One KDA decode step of one head: q, k, v bf16 bits [128]; alpha fp32 [128];
    S bf16 bits [128,128] (row = key channel).  Returns (new S bits, o [128] f64)."""
    q, k, v = _c(q, np.uint16), _c(k, np.uint16), _c(v, np.uint16)
    alpha = _c(alpha, np.float32)
    S = np.array(S, dtype=np.uint16, copy=True, order="C")
    o = np.empty(KDA_DIM, np.float64)
    rc = _load().oracle_kda_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), float(beta), _ptr(S), _ptr(o))
    if rc != 0:
        raise ValueError(f"oracle_kda_step rc={rc}")
    return S, o


def bf16_round(x: float) -> int:
    """Nearest bf16 (ties to even) of a double, as bits."""
    return int(_load().oracle_bf16_round(float(x)))


def map_rows(fn, items, threads: int | None = None):
    """Run fn over independent items on host threads; returns results in order."""
    items = list(items)
    nt = threads or n_threads()
    if nt == 1 or len(items) <= 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(nt) as ex:
        return list(ex.map(fn, items))
