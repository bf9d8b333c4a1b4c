"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare it with the float64 oracle on the same seeded inputs."""
from __future__ import annotations

import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import mamba2_tree_verification_amd as m
import oracle
from testgen import configs as C
from testgen.device import upload

RTOL, ATOL = 1e-4, 1e-5


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def assert_close(gpu, ref, what):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    bad = ~(np.abs(gpu - ref) <= ATOL + RTOL * np.abs(ref))
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, np.abs(gpu - ref), -1)), gpu.shape)
        raise AssertionError("%s: %d of %d outside tolerance; worst at %s gpu=%r ref=%r" %
                             (what, int(bad.sum()), bad.size, i, gpu[i], ref[i]))


def f32_bits_equal(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))


class GpuCase:
    """One workload on the GPU: inputs uploaded once, verify / commit runs."""

    def __init__(self, cfg, inp=None, device="cuda", fifo=False):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.inp = inp if inp is not None else C.make_inputs(cfg)
        self.g = upload(self.inp, device)
        self.dims = m.make_dims(cfg.L, cfg.Bsz, cfg.T, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.bf16, cfg.silu, fifo,
                                cfg.xbc, getattr(cfg, "state_bf16", False))
        self.prm = m.make_params(self.g.A, self.g.D, self.g.dt_bias, self.g.conv_w, self.g.conv_b)
        self.device = device

    def verify(self, y=None, fill=float("nan")):
        t, cfg = self.torch, self.cfg
        if y is None:
            y = t.full((cfg.L, cfg.Bsz, cfg.T, cfg.d_in), fill, dtype=t.float32, device=self.device)
        st = t.full((cfg.Bsz,), 12345, dtype=t.int32, device=self.device)
        g = self.g
        m.verify(self.dims, self.prm, g.parent, g.x, g.B, g.C, g.dt_raw, g.window, g.state, y, st, z=g.z)
        t.cuda.synchronize()
        return y, st

    def commit(self, inplace=False, state=None, window=None):
        t, g = self.torch, self.g
        st = t.full((self.cfg.Bsz,), 12345, dtype=t.int32, device=self.device)
        s_in = g.state if state is None else state
        w_in = g.window if window is None else window
        if inplace:
            s_out, w_out = s_in, w_in
        else:
            s_out = t.full_like(s_in, -777.0)
            w_out = None if w_in is None else t.zeros_like(w_in)
        m.commit(self.dims, self.prm, g.parent, g.path, g.path_len, g.x, g.B, g.dt_raw, w_in, s_in, w_out, s_out, st,
                 C=g.C if self.cfg.xbc else None)
        t.cuda.synchronize()
        return s_out, w_out, st

    # -- oracle side --------------------------------------------------------
    def oracle_verify(self, units, threads=16):
        return oracle.verify_units(self.cfg, self.inp, units, threads)

    def oracle_commit(self, units, threads=16):
        return oracle.commit_units(self.cfg, self.inp, units, threads)


def window_f64(cfg, w_tensor, l, b):
    """GPU window slice as float64 (exact) for comparison."""
    a = w_tensor[l, b]
    return a.float().double().cpu().numpy()


def check_verify(case, y, st, units):
    cfg = case.cfg
    ref = case.oracle_verify(units)
    stn = st.cpu().numpy()
    for (l, b), (yr, rc, _) in ref.items():
        assert stn[b] == rc, ("status", b, stn[b], rc)
        yg = y[l, b].double().cpu().numpy()
        if rc == 0:
            assert_close(yg, yr, "%s y[l=%d,b=%d]" % (cfg.name, l, b))
        else:
            assert np.isnan(yg).all()


def check_commit(case, s_out, w_out, st, units, untouched_state=None, untouched_window=None):
    cfg = case.cfg
    ref = case.oracle_commit(units)
    stn = st.cpu().numpy()
    for (l, b), (sr, wr, rc) in ref.items():
        assert stn[b] == rc, ("commit status", b, stn[b], rc)
        sg = s_out[l, b].double().cpu().numpy()
        if rc == 0:
            assert_close(sg, sr, "%s state[l=%d,b=%d]" % (cfg.name, l, b))
            if cfg.W > 1:
                wg = window_f64(cfg, w_out, l, b)
                assert np.array_equal(wg, wr), "window l=%d b=%d" % (l, b)
        else:
            if untouched_state is not None:
                assert np.array_equal(s_out[l, b].cpu().numpy(), untouched_state[l, b].cpu().numpy())
            if untouched_window is not None and cfg.W > 1:
                assert np.array_equal(w_out[l, b].float().cpu().numpy(), untouched_window[l, b].float().cpu().numpy())


def sample_units(cfg, k, rng, must=()):
    units = list(must)
    allu = [(l, b) for l in range(cfg.L) for b in range(cfg.Bsz)]
    if len(allu) <= k:
        return allu
    idx = rng.choice(len(allu), size=k, replace=False)
    for i in idx:
        if allu[i] not in units:
            units.append(allu[i])
    return units
