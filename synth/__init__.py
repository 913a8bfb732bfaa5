"""Seeded synthetic inputs for the sparse-attention path (shared by the oracle's
tests, the GPU tests and the benchmark; holds none of the method's arithmetic).

The generator itself is ``synth.c`` (counter-based SplitMix64; its header gives
the full definition).  This module compiles it with gcc on first use, exposes
thread-parallel wrappers (ctypes releases the GIL, and every element is a pure
function of (seed, tensor id, index), so chunks are independent), and builds
the five workloads' input tensors in ``synth.configs``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile synth.c into libsynth.so (plain gcc, no GPU code)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
            u64 = ctypes.c_uint64
            vp = ctypes.c_void_p
            lib.synth_normal_bf16.argtypes = [u64, u64, u64, u64, vp]
            lib.synth_normal_f64.argtypes = [u64, u64, u64, u64, vp]
            lib.synth_uniform_f64.argtypes = [u64, u64, u64, u64, vp]
            lib.synth_uniform_i8.argtypes = [u64, u64, u64, u64, ctypes.c_int32, ctypes.c_int32, vp]
            lib.synth_uniform_i64.argtypes = [u64, u64, u64, u64, ctypes.c_int64, ctypes.c_int64, vp]
            lib.synth_u64.argtypes = [u64, u64, u64, u64, vp]
            lib.synth_key.argtypes = [u64, u64]
            lib.synth_key.restype = u64
            for f in (lib.synth_normal_bf16, lib.synth_normal_f64, lib.synth_uniform_f64,
                      lib.synth_uniform_i8, lib.synth_uniform_i64, lib.synth_u64):
                f.restype = None
            _lib = lib
    return _lib


def n_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _parallel(fn, out: np.ndarray, start: int, extra=()):
    n = out.size
    flat = out.reshape(-1)
    chunk = 1 << 20
    if n <= chunk:
        fn(*extra[:2], start, n, *extra[2:], flat.ctypes.data)
        return out
    nt = n_threads()
    per = max(chunk, (n + nt * 4 - 1) // (nt * 4))
    ranges = [(i, min(n, i + per)) for i in range(0, n, per)]
    itemsize = flat.itemsize
    base = flat.ctypes.data

    def work(r):
        a, b = r
        fn(*extra[:2], start + a, b - a, *extra[2:], base + a * itemsize)

    with ThreadPoolExecutor(nt) as ex:
        list(ex.map(work, ranges))
    return out


def normal_bf16(seed: int, tensor: int, shape, start: int = 0) -> np.ndarray:
    """N(0,1) rounded to bf16; returns the raw bf16 bits as uint16."""
    out = np.empty(shape, dtype=np.uint16)
    return _parallel(_load().synth_normal_bf16, out, start, (seed, tensor))


def normal_f64(seed: int, tensor: int, shape, start: int = 0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float64)
    return _parallel(_load().synth_normal_f64, out, start, (seed, tensor))


def uniform_f64(seed: int, tensor: int, shape, start: int = 0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float64)
    return _parallel(_load().synth_uniform_f64, out, start, (seed, tensor))


def uniform_i8(seed: int, tensor: int, shape, lo: int, hi: int, start: int = 0) -> np.ndarray:
    """Integers uniform on [lo, hi] (both inclusive) as int8."""
    assert -128 <= lo <= hi <= 127
    out = np.empty(shape, dtype=np.int8)
    return _parallel(_load().synth_uniform_i8, out, start, (seed, tensor, lo, hi))


def uniform_i64(seed: int, tensor: int, shape, lo: int, hi: int, start: int = 0) -> np.ndarray:
    out = np.empty(shape, dtype=np.int64)
    return _parallel(_load().synth_uniform_i64, out, start, (seed, tensor, lo, hi))


def raw_u64(seed: int, tensor: int, shape, start: int = 0) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint64)
    return _parallel(_load().synth_u64, out, start, (seed, tensor))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)
