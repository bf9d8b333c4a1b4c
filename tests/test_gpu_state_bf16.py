"""bfloat16 root-state storage (SSM_TREE_STATE_BF16) against the float64 oracle.

The state is read exactly (bf16 -> float64 on the oracle side).  A committed
state is rounded to bfloat16 when stored; the oracle rounds its float64
result (oracle_round_bf16).  Near a rounding tie the float32 kernel and the
float64 oracle may fall on either side, so the test derives the admissible
stored values from the oracle alone: the bf16 roundings of every value within
the float32 parity band (atol 1e-5 + rtol 1e-4) of the exact state, i.e. the
grid points between round(h - t) and round(h + t).  The y of a round is
verified from the stored state; the oracle's y comes from its own rounding,
and a stored state anywhere in the band moves y_v[c] by at most
sum_n |C_v[n]| |dh[c][n]| (|exp(S_v)| <= 1 since A < 0 and dt > 0), which is
added to that element's tolerance.
"""
import numpy as np
import pytest
import torch

import mamba2_tree_verification_amd as m
import oracle
from testgen import configs as C
from tests.gpu_util import ATOL, RTOL, GpuCase, assert_close, log, window_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load()


def cfg_of(spec, cid):
    L, Bsz, T, H, P, N, G, W, bf16, silu, tree = spec
    return C.Config(cid, "sbf16", L, Bsz, T, H, P, N, G, W, bf16, 0.5, tree, silu, False, state_bf16=True)


# L, Bsz, T, H, P, N, G, W, bf16, silu, tree
VERIFY_SPECS = [
    (2, 3, 16, 8, 64, 128, 1, 4, True, False, "forest"),       # matrix cores, 16-node tiles
    (1, 4, 5, 4, 32, 16, 2, 3, True, True, "forest"),
    (2, 2, 13, 4, 64, 64, 1, 2, False, False, "forest"),       # fp32 inputs
    (1, 3, 40, 3, 64, 256, 3, 4, True, False, "forest"),       # 17-64 nodes, one single bf16 product
    (2, 2, 64, 2, 64, 128, 1, 4, True, True, "chain_or_star"),
    (1, 2, 33, 4, 64, 128, 1, 4, False, False, "forest"),      # 17-64 nodes, fp32 inputs
    (1, 3, 20, 8, 16, 16, 1, 4, True, True, "forest"),         # heads of 16 channels
    (1, 2, 48, 8, 64, 128, 1, 4, True, False, "forest"),       # 8 one-head blocks: the role-split kernel
    (1, 2, 64, 16, 64, 64, 1, 2, True, True, "chain_or_star"),  # 16 blocks; the round in one launch
    (1, 2, 33, 40, 64, 64, 1, 4, True, False, "forest"),       # 40 blocks per workgroup in verify
    # bf16 products over pairs of column groups (up to 16 nodes): d_state
    # 32, 64 (heads of 32 channels) and 256 (a ring of four pieces)
    (1, 3, 12, 4, 64, 32, 1, 4, True, False, "forest"),
    (2, 2, 9, 4, 32, 64, 2, 3, True, True, "forest"),
    (1, 2, 16, 2, 64, 256, 1, 4, True, True, "forest"),
]
COMMIT_SPECS = VERIFY_SPECS + [
    (1, 3, 12, 8, 40, 32, 1, 4, True, False, "forest"),        # headdim 40: commit takes every shape
]


def state_band(o, h):
    """Stored value expected (the oracle's rounding), the admissible range
    [lo, hi] on the bf16 grid, and the largest admissible deviation."""
    t = ATOL + RTOL * np.abs(h)
    r, _ = o.round_bf16(h)
    lo, _ = o.round_bf16(h - t)
    hi, _ = o.round_bf16(h + t)
    return r, lo, hi, np.maximum(hi - r, r - lo)


def check_state(g, h, o, what):
    r, lo, hi, dev = state_band(o, h)
    bad = ~((g >= lo) & (g <= hi))
    if bad.any():
        i = np.unravel_index(np.argmax(bad), g.shape)
        raise AssertionError("%s: %d of %d stored values outside the band; at %s gpu=%r exact=%r band=[%r, %r]" %
                             (what, int(bad.sum()), bad.size, i, g[i], h[i], lo[i], hi[i]))
    return r, dev


def y_extra(cfg, u, dev):
    """Per (node, channel) bound on how far y moves when the stored state
    ranges over its band: sum_n |C_v[g(c)][n]| dev[c][n]."""
    H, P, N, G = cfg.H, cfg.P, cfg.N, cfg.G
    devc = dev.reshape(H * P, N)
    ext = np.zeros((cfg.T, H * P))
    hpg = H // G
    for g in range(G):
        cs = slice(g * hpg * P, (g + 1) * hpg * P)
        ext[:, cs] = np.abs(u["C"][:, g, :]) @ devc[cs, :].T
    return ext


@pytest.mark.parametrize("spec", VERIFY_SPECS, ids=lambda s: "T%dH%dP%dN%dG%d%s" % (s[2], s[3], s[4], s[5], s[6],
                                                                                    "bf" if s[8] else "f32"))
def test_verify_state_bf16(spec):
    cfg = cfg_of(spec, 70 + VERIFY_SPECS.index(spec))
    log("verify with a bf16 state %s" % (spec,))
    case = GpuCase(cfg)
    assert case.g.state.dtype == torch.bfloat16
    y, st = case.verify()
    units = [(l, b) for l in range(cfg.L) for b in range(cfg.Bsz)]
    ref = case.oracle_verify(units)
    stn = st.cpu().numpy()
    for (l, b), (yr, rc, _) in ref.items():
        assert stn[b] == rc
        assert_close(y[l, b].double().cpu().numpy(), yr, "y l=%d b=%d" % (l, b))


@pytest.mark.parametrize("inplace", [False, True])
@pytest.mark.parametrize("spec", COMMIT_SPECS, ids=lambda s: "T%dH%dP%dN%dG%d%s" % (s[2], s[3], s[4], s[5], s[6],
                                                                                    "bf" if s[8] else "f32"))
def test_commit_state_bf16(spec, inplace):
    cfg = cfg_of(spec, 80 + COMMIT_SPECS.index(spec))
    log("commit with a bf16 state %s inplace=%s" % (spec, inplace))
    case = GpuCase(cfg)
    s_in = case.g.state.clone()
    w_in = None if case.g.window is None else case.g.window.clone()
    s_out, w_out, st = case.commit(inplace=inplace, state=s_in, window=w_in)
    assert s_out.dtype == torch.bfloat16
    o = oracle.get()
    units = [(l, b) for l in range(cfg.L) for b in range(cfg.Bsz)]
    ref = case.oracle_commit(units)
    stn = st.cpu().numpy()
    for (l, b), (sr, wr, rc) in ref.items():
        assert stn[b] == rc
        sg = s_out[l, b].double().cpu().numpy()
        if rc == 0:
            check_state(sg, sr, o, "state l=%d b=%d" % (l, b))
            if cfg.W > 1:
                assert np.array_equal(window_f64(cfg, w_out, l, b), wr)
        elif inplace:
            assert torch.equal(s_out[l, b].view(torch.int16), case.g.state[l, b].view(torch.int16))


def run_round(case, y=None):
    """One ssm_tree_commit_verify with the workload's tree as both the
    committed tree and the next tree (state and window out of place)."""
    cfg, g = case.cfg, case.g
    s_out = torch.full_like(g.state, -777.0)
    w_out = None if g.window is None else torch.zeros_like(g.window)
    y = torch.full((cfg.L, cfg.Bsz, cfg.T, cfg.d_in), float("nan"), dtype=torch.float32, device="cuda")
    cst = torch.full((cfg.Bsz,), 12345, dtype=torch.int32, device="cuda")
    vst = torch.full((cfg.Bsz,), 12345, dtype=torch.int32, device="cuda")
    m.commit_verify(case.dims, case.prm, g.parent, g.path, g.path_len, g.x, g.B, g.dt_raw, g.window, g.state, w_out,
                    s_out, g.parent, g.x, g.B, g.C, g.dt_raw, y, cst, vst)
    torch.cuda.synchronize()
    return s_out, w_out, y, cst, vst


def check_round(case, s_out, w_out, y, cst, vst, units):
    """The oracle's commit, its rounding to bf16, then its verify of the next
    tree from the rounded state and the committed window."""
    cfg = case.cfg
    o = oracle.get()
    cstn, vstn = cst.cpu().numpy(), vst.cpu().numpy()
    for (l, b) in units:
        u = C.unit_f64(cfg, l, b, case.inp)
        n = int(case.inp.path_len[b])
        so, wo, rc = o.commit(case.inp.parent[b], case.inp.path[b, :n], n, u, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W,
                              cfg.silu)
        assert cstn[b] == rc
        sg = s_out[l, b].double().cpu().numpy()
        if rc == 0:
            r, dev = check_state(sg, so, o, "round state l=%d b=%d" % (l, b))
        else:  # a failed commit passes the state through
            assert np.array_equal(sg, u["state"])
            r, dev = u["state"], np.zeros_like(u["state"])
        if cfg.W > 1:
            assert np.array_equal(window_f64(cfg, w_out, l, b), wo)
        un = dict(u, state=r, window=wo.reshape(u["window"].shape))
        yr, vrc, _ = o.verify(case.inp.parent[b], un, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.silu)
        assert vstn[b] == vrc
        yg = y[l, b].double().cpu().numpy()
        tol = ATOL + RTOL * np.abs(yr) + y_extra(cfg, u, dev)
        bad = ~(np.abs(yg - yr) <= tol)
        if bad.any():
            i = np.unravel_index(np.argmax(bad), yg.shape)
            raise AssertionError("round y l=%d b=%d: %d of %d outside; at %s gpu=%r ref=%r tol=%r" %
                                 (l, b, int(bad.sum()), bad.size, i, yg[i], yr[i], tol[i]))


@pytest.mark.parametrize("spec", VERIFY_SPECS, ids=lambda s: "T%dH%dP%dN%dG%d%s" % (s[2], s[3], s[4], s[5], s[6],
                                                                                    "bf" if s[8] else "f32"))
def test_round_state_bf16(spec):
    """The fused round (T <= 16), the one-launch round of the role-split
    verify (17-64 nodes, 8 or 16 one-head blocks per B/C group) and the
    two-call form (other 17-64-node shapes)."""
    cfg = cfg_of(spec, 90 + VERIFY_SPECS.index(spec))
    log("round with a bf16 state %s" % (spec,))
    case = GpuCase(cfg)
    s_out, w_out, y, cst, vst = run_round(case)
    check_round(case, s_out, w_out, y, cst, vst, [(l, b) for l in range(cfg.L) for b in range(cfg.Bsz)])
    # the round verifies from exactly the state it stored: the same y as a
    # separate verify from that stored state (a property of the GPU path, in
    # addition to the oracle check above, whose band allows either rounding)
    g = case.g
    y2 = torch.full_like(y, float("nan"))
    m.verify(case.dims, case.prm, g.parent, g.x, g.B, g.C, g.dt_raw, w_out, s_out, y2)
    torch.cuda.synchronize()
    assert_close(y.double().cpu().numpy(), y2.double().cpu().numpy(), "round y vs verify from the stored state")


def test_round_state_bf16_full_size():
    """The 2.7B batch-16 tree-16 workload with a bf16 state, sampled units."""
    cfg = C.CONFIGS[3].replace(state_bf16=True)
    log("round with a bf16 state on %s" % cfg.name)
    case = GpuCase(cfg)
    s_out, w_out, y, cst, vst = run_round(case)
    rng = np.random.default_rng(7)
    units = [(cfg.L - 1, cfg.Bsz - 1), (0, 0)] + [(int(rng.integers(cfg.L)), int(rng.integers(cfg.Bsz)))
                                                for _ in range(4)]
    check_round(case, s_out, w_out, y, cst, vst, units)


def test_round_state_bf16_failures():
    """An invalid previous path passes the state through untouched; an
    invalid next tree gives NaN y and its status."""
    cfg = cfg_of((1, 4, 12, 4, 64, 64, 1, 4, True, False, "forest"), 99)
    inp = C.make_inputs(cfg)
    inp.path_len[1] = cfg.T + 1          # over-long path: commit fails for sequence 1
    case = GpuCase(cfg, inp)
    s_out, w_out, y, cst, vst = run_round(case)
    cstn = cst.cpu().numpy()
    assert cstn[1] == m.E_PATH and (cstn[[0, 2, 3]] == m.OK).all()
    check_round(case, s_out, w_out, y, cst, vst, [(0, b) for b in range(cfg.Bsz)])


@pytest.mark.parametrize("spec", [(2, 3, 16, 8, 64, 128, 1, 4, True, True, "forest"),
                                  (1, 4, 40, 4, 32, 64, 2, 3, False, False, "chain_or_star")],
                         ids=["T16bf", "T40f32"])
def test_commit_bf16_store_rounds_the_fp32_commit(spec):
    """The commit's arithmetic is float32 whatever the stored state type, so
    a bf16-state commit must store exactly the round-to-nearest-even of what
    the float32-state commit computes from the same (widened) state: the
    device rounding checked bit for bit against the oracle's rounding."""
    cfg = cfg_of(spec, 112 + (spec[2] == 40))
    log("bf16 store vs rounded fp32 commit %s" % (spec,))
    case = GpuCase(cfg)
    g = case.g
    s_bf = torch.empty_like(g.state)
    w_bf = torch.empty_like(g.window)
    st_bf = torch.empty((cfg.Bsz,), dtype=torch.int32, device="cuda")
    m.commit(case.dims, case.prm, g.parent, g.path, g.path_len, g.x, g.B, g.dt_raw, g.window, g.state, w_bf, s_bf,
             st_bf)
    dims32 = m.make_dims(cfg.L, cfg.Bsz, cfg.T, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.bf16, cfg.silu)
    s32_in = g.state.float()
    s32 = torch.empty_like(s32_in)
    w32 = torch.empty_like(g.window)
    st32 = torch.empty_like(st_bf)
    m.commit(dims32, case.prm, g.parent, g.path, g.path_len, g.x, g.B, g.dt_raw, g.window, s32_in, w32, s32, st32)
    torch.cuda.synchronize()
    assert torch.equal(st_bf, st32) and (st32.cpu().numpy() == 0).all()
    assert torch.equal(w_bf, w32)
    r, _ = oracle.get().round_bf16(s32.double().cpu().numpy())
    assert np.array_equal(s_bf.double().cpu().numpy(), r)
