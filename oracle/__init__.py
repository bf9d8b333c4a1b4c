"""ctypes wrapper of the float64 C oracle (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP
library; it receives float64 copies of exactly the values the GPU receives.
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
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_libs: dict = {}

OK, E_ARG, E_TREE, E_PATH = 0, -3, -10, -11
PLAN_STRIDE = 8
PLAN_UNUSED = -32768


def build(force: bool = True, mutant: int = 0, out: str | None = None) -> str:
    """Compile the oracle with gcc (plain C99).  `mutant` plants one mistake."""
    target = out or _LIB
    if force or not os.path.exists(target):
        tmp = target + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
               "-DORACLE_MUTANT=%d" % mutant, "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, target)
    return target


class _Dims(ctypes.Structure):
    _fields_ = [(k, ctypes.c_int32) for k in ("T", "H", "P", "N", "G", "W", "silu", "xbc")]


class _Unit(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in
                ("x", "B", "C", "dt_raw", "window", "state", "A", "D", "dt_bias", "conv_w", "conv_b", "z")]


class Oracle:
    """One loaded copy of the oracle library (the real one or a mutant)."""

    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        p, i32 = ctypes.c_void_p, ctypes.c_int32
        L.oracle_validate_tree.argtypes = [p, i32]
        L.oracle_validate_path.argtypes = [p, i32, p, i32]
        L.oracle_plan.argtypes = [p, i32, i32, p, p, p, p]
        L.oracle_verify.argtypes = [p, p, p, p, p]
        L.oracle_commit.argtypes = [p, p, p, i32, p, p, p]
        L.oracle_scan.argtypes = [p, i32, p, p, p, p]
        L.oracle_round_bf16.argtypes = [p, p, p, ctypes.c_int64]
        L.oracle_round_bf16.restype = None
        for f in ("oracle_validate_tree", "oracle_validate_path", "oracle_plan", "oracle_verify",
                  "oracle_commit", "oracle_scan"):
            getattr(L, f).restype = ctypes.c_int
        self.lib = L
        self.path = path

    # -- helpers ------------------------------------------------------------
    @staticmethod
    def _dims(T, H, P, N, G, W, silu, xbc=False):
        return _Dims(T, H, P, N, G, W, int(bool(silu)), int(bool(xbc)))

    @staticmethod
    def conv_channels(H, P, N, G, xbc=False):
        """Channels of the causal conv: x, or x, B and C with xbc."""
        return H * P + (2 * G * N if xbc else 0)

    @staticmethod
    def _unit(u: dict, keep: list):
        def ptr(k):
            a = u.get(k)
            if a is None:
                return None
            a = np.ascontiguousarray(a, dtype=np.float64)
            keep.append(a)
            return a.ctypes.data
        return _Unit(*(ptr(k) for k in ("x", "B", "C", "dt_raw", "window", "state", "A", "D",
                                          "dt_bias", "conv_w", "conv_b", "z")))

    @staticmethod
    def _i32(a):
        return np.ascontiguousarray(a, dtype=np.int32)

    # -- API ----------------------------------------------------------------
    def validate_tree(self, parent) -> int:
        p = self._i32(parent)
        return self.lib.oracle_validate_tree(p.ctypes.data, len(p))

    def validate_path(self, parent, path, length) -> int:
        p, q = self._i32(parent), self._i32(path)
        if len(q) == 0:
            q = np.zeros(1, np.int32)
        return self.lib.oracle_validate_path(p.ctypes.data, len(p), q.ctypes.data, int(length))

    def plan(self, parent, W):
        p = self._i32(parent)
        T = len(p)
        out = np.zeros((max(T, 1), PLAN_STRIDE), np.int32)
        pk, md, ni = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
        st = self.lib.oracle_plan(p.ctypes.data, T, W, out.ctypes.data, ctypes.byref(pk),
                                  ctypes.byref(md), ctypes.byref(ni))
        return st, out[:T], dict(peak_fifo=pk.value, max_depth=md.value, n_internal=ni.value)

    def verify(self, parent, u: dict, H, P, N, G, W, silu=False, xbc=False):
        """y [T][H*P] float64, status, peak FIFO occupancy for one unit.
        u["z"] (optional) gates y by silu(z); xbc convolves B and C too."""
        p = self._i32(parent)
        T = len(p)
        keep: list = []
        y = np.zeros((T, H * P), np.float64)
        pk = ctypes.c_int32(0)
        d = self._dims(T, H, P, N, G, W, silu, xbc)
        st = self.lib.oracle_verify(ctypes.byref(d), p.ctypes.data if T else None,
                                    ctypes.byref(self._unit(u, keep)), y.ctypes.data, ctypes.byref(pk))
        return y, st, pk.value

    def commit(self, parent, path, length, u: dict, H, P, N, G, W, silu=False, xbc=False):
        """(state_out [H][P][N], window_out [W-1][CH], status).  Outputs are
        copies of the inputs when the status is not OK (the oracle leaves its
        output buffers untouched, and they start as copies here)."""
        p = self._i32(parent)
        q = self._i32(path)
        T = len(p)
        if len(q) == 0:
            q = np.zeros(1, np.int32)
        keep: list = []
        CH = self.conv_channels(H, P, N, G, xbc)
        so = np.array(u["state"], dtype=np.float64, copy=True)
        wo = np.array(u["window"], dtype=np.float64, copy=True).reshape(max(W - 1, 0), CH)
        d = self._dims(T, H, P, N, G, W, silu, xbc)
        st = self.lib.oracle_commit(ctypes.byref(d), p.ctypes.data if T else None, q.ctypes.data,
                                    int(length), ctypes.byref(self._unit(u, keep)), so.ctypes.data,
                                    wo.ctypes.data if W > 1 else None)
        return so, wo, st

    def round_bf16(self, x):
        """Storage rounding of a committed state to bfloat16 (oracle.h):
        (rounded values as float64, distance to the nearest rounding
        boundary relative to |x|), both shaped like x."""
        a = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty_like(a)
        gap = np.empty_like(a)
        self.lib.oracle_round_bf16(a.ctypes.data, out.ctypes.data, gap.ctypes.data, a.size)
        return out, gap

    def scan(self, u: dict, S, H, P, N, G, W, silu=False, xbc=False):
        """Plain sequential scan of S tokens: (y [S][H*P], state_out, window_out [W-1][CH])."""
        keep: list = []
        y = np.zeros((S, H * P), np.float64)
        so = np.zeros((H, P, N), np.float64)
        wo = np.zeros((max(W - 1, 0), self.conv_channels(H, P, N, G, xbc)), np.float64)
        d = self._dims(0, H, P, N, G, W, silu, xbc)
        st = self.lib.oracle_scan(ctypes.byref(d), S, ctypes.byref(self._unit(u, keep)), y.ctypes.data,
                                  so.ctypes.data, wo.ctypes.data if W > 1 else None)
        assert st == OK, st
        return y, so, wo


def get(mutant: int = 0) -> Oracle:
    """The oracle library (built on first use if absent); mutants are built
    into a temporary path on demand."""
    with _lock:
        if mutant in _libs:
            return _libs[mutant]
        if mutant == 0:
            if not os.path.exists(_LIB):
                build(force=False)
            path = _LIB
        else:
            import tempfile
            d = tempfile.mkdtemp(prefix="oracle_mut%d_" % mutant)
            path = build(force=True, mutant=mutant, out=os.path.join(d, "liboracle_mut.so"))
        o = Oracle(path)
        _libs[mutant] = o
        return o


def verify_units(cfg, inputs, units, threads: int = 8, oracle: Oracle | None = None):
    """Run the oracle's verify on several (layer, sequence) units in threads.

    Returns {(l, b): (y [T][d_in], status, peak)}.  ctypes releases the GIL,
    so the units run in parallel."""
    from testgen.configs import unit_f64
    o = oracle or get()

    def one(lb):
        l, b = lb
        u = unit_f64(cfg, l, b, inputs)
        return lb, o.verify(inputs.parent[b] if inputs is not None else None, u, cfg.H, cfg.P, cfg.N,
                            cfg.G, cfg.W, cfg.silu, getattr(cfg, "xbc", False))

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        return dict(ex.map(one, units))


def commit_units(cfg, inputs, units, threads: int = 8, oracle: Oracle | None = None):
    from testgen.configs import unit_f64
    o = oracle or get()

    def one(lb):
        l, b = lb
        u = unit_f64(cfg, l, b, inputs)
        n = int(inputs.path_len[b])
        return lb, o.commit(inputs.parent[b], inputs.path[b, :n], n, u, cfg.H, cfg.P, cfg.N, cfg.G,
                            cfg.W, cfg.silu, getattr(cfg, "xbc", False))

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        return dict(ex.map(one, units))
