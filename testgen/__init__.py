"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module is the only code that both sides of a parity check use, and it
holds none of the SSM arithmetic: tensors come from a counter-based
generator written in C (``testgen.c``: SplitMix64 mixing plus the
Box-Muller transform), trees and accepted paths from numpy's PCG64 stream.
A value depends only on (seed, stream id, flat element index), so any
(layer, sequence) slice of a large tensor can be regenerated on its own.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "testgen.c")
_LIB = os.path.join(_HERE, "libtestgen.so")
_lock = threading.Lock()
_lib = None

DIST_NORMAL, DIST_UNIFORM, DIST_NEG_EXP_UNIFORM = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile libtestgen.so in place with gcc (plain C99, pthreads)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-fPIC", "-shared",
               "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=False)
            L = ctypes.CDLL(_LIB)
            i64, u64, dbl, ci = ctypes.c_int64, ctypes.c_uint64, ctypes.c_double, ctypes.c_int
            L.tg_fill_f32.argtypes = [ctypes.c_void_p, i64, u64, u64, i64, ci, dbl, dbl, ci]
            L.tg_fill_f32.restype = ci
            L.tg_fill_bf16.argtypes = [ctypes.c_void_p, i64, u64, u64, i64, ci, dbl, dbl, ci]
            L.tg_fill_bf16.restype = ci
            L.tg_raw_bits.argtypes = [ctypes.c_void_p, i64, u64, u64, i64]
            L.tg_raw_bits.restype = None
            L.tg_f32_to_bf16.argtypes = [ctypes.c_float]
            L.tg_f32_to_bf16.restype = ctypes.c_uint16
            _lib = L
    return _lib


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def fill(shape, seed: int, stream: int, dist: int, a: float, b: float, bf16: bool,
         offset: int = 0, nthreads: int | None = None) -> np.ndarray:
    """Draw a tensor; bf16 tensors are returned as their raw uint16 bit patterns."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(shape, dtype=np.uint16 if bf16 else np.float32)
    nt = default_threads() if nthreads is None else nthreads
    f = lib().tg_fill_bf16 if bf16 else lib().tg_fill_f32
    f(out.ctypes.data, n, seed & 0xFFFFFFFFFFFFFFFF, stream, offset, dist, a, b, nt)
    return out


def raw_bits(n: int, seed: int, stream: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    lib().tg_raw_bits(out.ctypes.data, n, seed, stream, offset)
    return out


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(u16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16 bit patterns (NaN kept quiet)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = ((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def as_f64(a: np.ndarray, is_bf16: bool) -> np.ndarray:
    """Exact float64 view of what the GPU receives."""
    if is_bf16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)
