"""GPU parity of ssm_tree_commit_verify: the commit of one tree's accepted
path followed by the verification of the next tree from the committed state
and window (one decode step of the speculative loop, SpecMamba page
sec. 3.1-3.2), against the float64 oracle's commit followed by its verify.

Trees of 1..16 nodes with headdim % 16 == 0 take the fused kernel; trees
of 17..64 nodes with bf16 inputs, d_state <= 128, heads a multiple of 64
channels and B/C groups of a multiple of 512 channels take the one-launch
round of the 17-64-node verify; other shapes, the options on 17-64 nodes
and the FIFO flag take the two calls in turn.  All are covered.
Tolerance as elsewhere: |gpu - oracle| <= 1e-5 + 1e-4 |oracle| for y and
the committed state; statuses and windows exactly.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mamba2_tree_verification_amd as m  # noqa: E402
import oracle  # noqa: E402
from testgen import as_f64  # noqa: E402
from testgen import configs as C  # noqa: E402
from testgen.device import tensor, upload  # noqa: E402
from tests.gpu_util import assert_close, log, sample_units, window_f64  # noqa: E402
from tests.test_gpu_parity import SMALL  # noqa: E402

pytestmark = pytest.mark.gpu

NEXT_ONLY = ("state", "window", "A", "D", "dt_bias", "conv_w", "conv_b")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load()


def fused_applies(cfg):
    return 1 <= cfg.T <= 16 and cfg.P % 16 == 0


def tt_round_applies(cfg, gate=False):
    """The one-launch round of trees of 17..64 nodes."""
    return (cfg.bf16 and 16 < cfg.T <= 64 and cfg.N <= 128 and cfg.P % 64 == 0 and (cfg.H * cfg.P // cfg.G) % 512 == 0
            and not cfg.xbc and not gate)


def route(cfg):
    return "fused" if fused_applies(cfg) else ("one launch, 17-64 nodes" if tt_round_applies(cfg) else "two calls")


class Step:
    """Previous tree (with its accepted path, root state, window and the
    layer parameters) and the next tree (nodes only), on the GPU."""

    def __init__(self, cfg, next_cid=None, prev=None, nxt=None, fifo=False):
        self.cfg = cfg
        self.prev = prev if prev is not None else C.make_inputs(cfg)
        self.ncfg = cfg.replace(cid=cfg.cid + 500 if next_cid is None else next_cid)
        self.nxt = nxt if nxt is not None else C.make_inputs(self.ncfg, skip=NEXT_ONLY)
        self.gp = upload(self.prev)
        self.gn = self._upload_next(self.nxt)
        self.dims = m.make_dims(cfg.L, cfg.Bsz, cfg.T, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.bf16, cfg.silu, fifo,
                                cfg.xbc)
        g = self.gp
        self.prm = m.make_params(g.A, g.D, g.dt_bias, g.conv_w, g.conv_b)

    def _upload_next(self, nxt):
        from types import SimpleNamespace
        ns = SimpleNamespace()
        ns.parent = torch.from_numpy(np.ascontiguousarray(nxt.parent, np.int32)).cuda()
        for k in ("x", "B", "C", "dt_raw", "z"):
            setattr(ns, k, tensor(getattr(nxt, k), self.cfg.bf16))
        return ns

    def run(self, inplace=False, state=None, window=None, y=None):
        cfg, gp, gn = self.cfg, self.gp, self.gn
        s_in = gp.state if state is None else state
        w_in = gp.window if window is None else window
        if inplace:
            s_out, w_out = s_in, w_in
        else:
            s_out = torch.full_like(s_in, -777.0)
            w_out = None if w_in is None else torch.zeros_like(w_in)
        if y is None:
            y = torch.full((cfg.L, cfg.Bsz, cfg.T, cfg.d_in), float("nan"), dtype=torch.float32, device="cuda")
        cst = torch.full((cfg.Bsz,), 12345, dtype=torch.int32, device="cuda")
        vst = torch.full((cfg.Bsz,), 12345, dtype=torch.int32, device="cuda")
        m.commit_verify(self.dims, self.prm, gp.parent, gp.path, gp.path_len, gp.x, gp.B, gp.dt_raw, w_in, s_in,
                        w_out, s_out, gn.parent, gn.x, gn.B, gn.C, gn.dt_raw, y, cst, vst,
                        C_prev=gp.C if cfg.xbc else None, z=gn.z)
        torch.cuda.synchronize()
        return s_out, w_out, y, cst, vst

    # -- oracle side --------------------------------------------------------
    def next_unit(self, l, b, state, window, params):
        shp = C.unit_shapes(self.cfg)
        u = dict(params)
        for k in ("x", "B", "C", "dt_raw", "z"):
            if getattr(self.nxt, k) is None:
                u[k] = None
                continue
            u[k] = as_f64(getattr(self.nxt, k)[l, b], self.cfg.bf16).reshape(shp[k])
        u["state"] = state
        u["window"] = window
        return u

    def oracle(self, units, threads=16):
        """{(l, b): (state_out, window_out, commit status, y, verify status)}."""
        cfg, prev, nxt = self.cfg, self.prev, self.nxt
        o = oracle.get()
        a = (cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.silu, cfg.xbc)

        def one(lb):
            l, b = lb
            u = C.unit_f64(cfg, l, b, prev)
            n = int(prev.path_len[b])
            so, wo, cst = o.commit(prev.parent[b], prev.path[b, :n], n, u, *a)
            y, vst, _ = o.verify(nxt.parent[b], self.next_unit(l, b, so, wo, u), *a)
            return lb, (so, wo, cst, y, vst)

        with ThreadPoolExecutor(max_workers=threads) as ex:
            return dict(ex.map(one, units))


def check(step, out, units, state_in=None, window_in=None):
    s_out, w_out, y, cst, vst = out
    cfg = step.cfg
    ref = step.oracle(units)
    cs, vs = cst.cpu().numpy(), vst.cpu().numpy()
    s_in = step.gp.state if state_in is None else state_in
    w_in = step.gp.window if window_in is None else window_in
    for (l, b), (so, wo, rc, yr, rv) in ref.items():
        assert cs[b] == rc, ("commit status", b, cs[b], rc)
        assert vs[b] == rv, ("verify status", b, vs[b], rv)
        if rc == 0:
            assert_close(s_out[l, b].double().cpu().numpy(), so, "%s state[l=%d,b=%d]" % (cfg.name, l, b))
        else:  # passed through bit for bit
            assert torch.equal(s_out[l, b].view(torch.int32), s_in[l, b].view(torch.int32)), (l, b)
        if cfg.W > 1:
            assert np.array_equal(window_f64(cfg, w_out, l, b), wo), "window l=%d b=%d" % (l, b)
            if rc != 0:
                assert torch.equal(w_out[l, b].view(torch.int16 if cfg.bf16 else torch.int32),
                                   w_in[l, b].view(torch.int16 if cfg.bf16 else torch.int32))
        yg = y[l, b].double().cpu().numpy()
        if rv == 0:
            assert_close(yg, yr, "%s y[l=%d,b=%d]" % (cfg.name, l, b))
        else:
            assert np.isnan(yg).all()


# ----------------------------------------------------------------------------
# the five workloads at full size (the 64-node stress trees take the one-launch
# round of the 17-64-node verify)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("cid,k", [(0, 1), (1, 4), (2, 4), (3, 6), (4, 3)])
def test_commit_verify_full_size(cid, k):
    cfg = C.CONFIGS[cid]
    log("commit_verify config %d %s (%s)" % (cid, cfg.name, route(cfg)))
    step = Step(cfg)
    out = step.run()
    assert not torch.isnan(out[2]).any(), "NaN in y"
    rng = np.random.default_rng(300 + cid)
    units = sample_units(cfg, k, rng, [(cfg.L - 1, cfg.Bsz - 1), (0, 0)])
    log("commit_verify config %d: oracle on %d units" % (cid, len(units)))
    check(step, out, units)


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: "L%dB%dT%dH%dP%dN%dG%dW%d%s%s%s" % (
    s[0], s[1], s[2], s[3], s[4], s[5], s[6], s[7], "bf" if s[8] else "f32", "S" if s[9] else "",
    "b" if s[10] else ""))
def test_commit_verify_small_random(spec):
    L, Bsz, T, H, P, N, G, W, bf16, silu, bias, tree = spec
    cfg = C.Config(110 + SMALL.index(spec), "small", L, Bsz, T, H, P, N, G, W, bf16, 0.5, tree, silu, bias)
    log("commit_verify small %s (%s)" % (spec, route(cfg)))
    step = Step(cfg)
    check(step, step.run(), [(l, b) for l in range(L) for b in range(Bsz)])


# ----------------------------------------------------------------------------
# failures, in place, agreement with the separate calls, a multi-step loop
# ----------------------------------------------------------------------------

def _edge_cfg(**kw):
    return C.Config(130, "edge", 2, 6, 12, 4, 64, 128, 1, 4, True, 0.5, "forest").replace(**kw)


@pytest.mark.parametrize("kw", [dict(), dict(T=24), dict(T=24, H=8), dict(P=40, H=8)],
                         ids=["fused", "T24", "T24-one-launch", "P40"])
@pytest.mark.parametrize("inplace", [False, True])
def test_failed_commits_pass_state_through(kw, inplace):
    cfg = _edge_cfg(**kw)
    log("failed commits %s (%s)" % (kw, route(cfg)))
    prev = C.make_inputs(cfg)
    prev.parent[1, 3] = 5                      # previous tree invalid (forward reference)
    prev.path_len[2] = cfg.T + 1               # path too long
    v = int(np.nonzero(prev.parent[3] >= 0)[0][0])
    prev.path[3, :2] = [v, 0]                  # first step not a root-level node
    prev.path_len[3] = 2
    step = Step(cfg, prev=prev)
    step.nxt.parent[4, 2] = -2                 # next tree invalid
    step.gn.parent.copy_(torch.from_numpy(step.nxt.parent))
    s_in, w_in = step.gp.state.clone(), step.gp.window.clone()
    out = step.run(inplace=inplace, state=s_in if inplace else None, window=w_in if inplace else None)
    cs, vs = out[3].cpu().numpy(), out[4].cpu().numpy()
    assert list(cs[1:4]) == [m.E_TREE, m.E_PATH, m.E_PATH], cs
    assert vs[4] == m.E_TREE and (np.delete(vs, 4) == 0).all(), vs
    check(step, out, [(l, b) for l in range(cfg.L) for b in range(cfg.Bsz)], state_in=step.gp.state,
          window_in=step.gp.window)


@pytest.mark.parametrize("kw", [dict(), dict(T=40, H=8)], ids=["fused", "one-launch-17-64"])
def test_inplace_equals_out_of_place(kw):
    cfg = _edge_cfg(**kw)
    step = Step(cfg)
    ref = step.run()
    s_in, w_in = step.gp.state.clone(), step.gp.window.clone()
    out = step.run(inplace=True, state=s_in, window=w_in)
    assert out[0].data_ptr() == s_in.data_ptr()
    for a, b in zip(ref, out):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b)


@pytest.mark.parametrize("kw", [dict(), dict(bf16=False, silu=True, conv_bias=True, N=64, W=3), dict(T=33, H=8),
                                dict(T=64, H=8, N=64, W=2, silu=True, conv_bias=True, tree="chain_or_star")])
def test_fused_agrees_with_separate_calls(kw):
    cfg = _edge_cfg(**kw)
    log("one round against commit then verify %s (%s)" % (kw, route(cfg)))
    step = Step(cfg)
    s_f, w_f, y_f, cs_f, vs_f = step.run()
    gp, gn = step.gp, step.gn
    s_c = torch.empty_like(gp.state)
    w_c = torch.empty_like(gp.window) if gp.window is not None else None
    cs = torch.empty((cfg.Bsz,), dtype=torch.int32, device="cuda")
    vs = torch.empty_like(cs)
    y = torch.empty_like(y_f)
    m.commit(step.dims, step.prm, gp.parent, gp.path, gp.path_len, gp.x, gp.B, gp.dt_raw, gp.window, gp.state,
             w_c, s_c, cs)
    m.verify(step.dims, step.prm, gn.parent, gn.x, gn.B, gn.C, gn.dt_raw, w_c, s_c, y, vs)
    torch.cuda.synchronize()
    assert torch.equal(cs, cs_f) and torch.equal(vs, vs_f)
    if w_c is not None:
        assert torch.equal(w_c, w_f)
    assert_close(s_f.double().cpu().numpy(), s_c.double().cpu().numpy(), "state fused vs separate")
    assert_close(y_f.double().cpu().numpy(), y.double().cpu().numpy(), "y fused vs separate")


def test_fifo_flag_takes_the_two_calls():
    cfg = _edge_cfg(Bsz=3)
    a = Step(cfg).run()
    b = Step(cfg, fifo=True).run()
    assert torch.equal(a[1], b[1]) and torch.equal(a[3], b[3]) and torch.equal(a[4], b[4])
    assert_close(b[0].double().cpu().numpy(), a[0].double().cpu().numpy(), "state fifo vs fused")
    assert_close(b[2].double().cpu().numpy(), a[2].double().cpu().numpy(), "y fifo vs fused")


@pytest.mark.parametrize("T,H", [(16, 4), (20, 4), (40, 8)])
def test_three_tree_loop(T, H):
    """Tree 1 -> (commit 1, verify 2) -> (commit 2, verify 3): the state
    carried on the GPU in place through two rounds equals the oracle's
    commit / verify chain."""
    cfg = _edge_cfg(Bsz=4, T=T, H=H)
    log("three-tree loop T=%d H=%d (%s)" % (T, H, route(cfg)))
    s1 = Step(cfg, next_cid=901)
    st, win = s1.gp.state.clone(), s1.gp.window.clone()
    s1.run(inplace=True, state=st, window=win)
    # step 2: tree 2 (with its own accepted path) is now the previous tree
    t2 = C.make_inputs(s1.ncfg)
    for k in NEXT_ONLY:  # the layer parameters stay those of step 1
        setattr(t2, k, getattr(s1.prev, k))
    s2 = Step(cfg, next_cid=902, prev=t2)
    out = s2.run(inplace=True, state=st, window=win)
    # oracle chain
    o = oracle.get()
    a = (cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.silu)
    for l in range(cfg.L):
        for b in range(cfg.Bsz):
            u1 = C.unit_f64(cfg, l, b, s1.prev)
            n1 = int(s1.prev.path_len[b])
            so1, wo1, c1 = o.commit(s1.prev.parent[b], s1.prev.path[b, :n1], n1, u1, *a)
            u2 = s1.next_unit(l, b, so1, wo1, u1)
            n2 = int(t2.path_len[b])
            so2, wo2, c2 = o.commit(t2.parent[b], t2.path[b, :n2], n2, u2, *a)
            y3, v3, _ = o.verify(s2.nxt.parent[b], s2.next_unit(l, b, so2, wo2, u1), *a)
            assert c1 == 0 and c2 == 0 and v3 == 0
            assert_close(out[0][l, b].double().cpu().numpy(), so2, "state after two steps l=%d b=%d" % (l, b))
            assert np.array_equal(window_f64(cfg, out[1], l, b), wo2)
            assert_close(out[2][l, b].double().cpu().numpy(), y3, "y of tree 3 l=%d b=%d" % (l, b))


def test_zero_sizes():
    for kw in (dict(L=0), dict(Bsz=0), dict(T=0)):
        cfg = _edge_cfg(**kw)
        step = Step(cfg)
        s_out, w_out, y, cs, vs = step.run()
        if cfg.L and cfg.Bsz:  # T = 0: nothing to commit, the state and window pass through
            assert torch.equal(s_out, step.gp.state) and torch.equal(w_out, step.gp.window)
            assert (cs.cpu().numpy() == 0).all() and (vs.cpu().numpy() == 0).all()


@pytest.mark.parametrize("kw", [dict(), dict(T=20), dict(T=20, H=8)], ids=["fused", "two-calls", "one-launch-17-64"])
def test_graph_replay_equals_eager(kw):
    """One round captured in a HIP graph (in place on the state and window)
    and replayed three times, with unrelated eager work and synchronisation
    between replays, equals three eager rounds bit for bit after every
    replay."""
    cfg = _edge_cfg(Bsz=3, **kw)
    step = Step(cfg)
    s0, w0 = step.gp.state.clone(), step.gp.window.clone()
    st, win = s0.clone(), w0.clone()
    y = torch.empty((cfg.L, cfg.Bsz, cfg.T, cfg.d_in), dtype=torch.float32, device="cuda")
    eager = []
    for _ in range(3):
        out = step.run(inplace=True, state=st, window=win, y=y)
        eager.append([t.clone() for t in out])
    st.copy_(s0)
    win.copy_(w0)
    y.fill_(0.0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    gp, gn = step.gp, step.gn
    cst = torch.empty((cfg.Bsz,), dtype=torch.int32, device="cuda")
    vst = torch.empty_like(cst)
    with torch.cuda.graph(graph, stream=side):
        m.commit_verify(step.dims, step.prm, gp.parent, gp.path, gp.path_len, gp.x, gp.B, gp.dt_raw, win, st, win,
                        st, gn.parent, gn.x, gn.B, gn.C, gn.dt_raw, y, cst, vst)
    torch.cuda.synchronize()
    assert torch.equal(st, s0), "capture must not execute the round"
    for r in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip((st, win, y, cst, vst), eager[r]):
            assert torch.equal(got.view(torch.int32) if got.dtype == torch.float32 else got,
                               ref.view(torch.int32) if ref.dtype == torch.float32 else ref), ("replay", r)
        junk = torch.randn(1 << 20, device="cuda")  # unrelated eager work between replays
        assert torch.isfinite(junk.sum())
        torch.cuda.synchronize()


def _token(t, k):
    """Node k of a [L][Bsz][T][...] tensor as a one-node tree [L][Bsz][1][...]."""
    return t[:, :, k:k + 1].contiguous()


@pytest.mark.parametrize("bf16", [True, False])
def test_draft_decode_then_rollback(bf16):
    """The draft side of speculative decoding (SpecMamba page sec. 3.1): K
    tokens decoded one at a time, each step a one-node round that commits
    the previous token into a working state and emits the new token's y;
    their x, B, dt_raw stay in a per-token log.  Rollback is a commit of
    the accepted prefix of the chain from the root state.  Both against the
    oracle's plain sequential scan."""
    K = 7
    cfg = C.Config(140, "draft", 3, 2, K, 8, 64, 128, 1, 4, bf16, 0.5, "chain")
    log_inp = C.make_inputs(cfg)  # the log: a chain of K tokens per sequence
    g = upload(log_inp)
    dims1 = m.make_dims(cfg.L, cfg.Bsz, 1, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.bf16)
    prm = m.make_params(g.A, g.D, g.dt_bias, g.conv_w, None)
    one = torch.tensor([[-1]] * cfg.Bsz, dtype=torch.int32, device="cuda")
    path0 = torch.zeros((cfg.Bsz, 1), dtype=torch.int32, device="cuda")
    work_s, work_w = torch.empty_like(g.state), torch.empty_like(g.window)
    cst = torch.empty((cfg.Bsz,), dtype=torch.int32, device="cuda")
    vst = torch.empty_like(cst)
    ys = []
    for k in range(K):
        plen = torch.full((cfg.Bsz,), 1 if k else 0, dtype=torch.int32, device="cuda")
        kp = max(k - 1, 0)
        y = torch.empty((cfg.L, cfg.Bsz, 1, cfg.d_in), dtype=torch.float32, device="cuda")
        s_in, w_in = (g.state, g.window) if k == 0 else (work_s, work_w)
        m.commit_verify(dims1, prm, one, path0, plen, _token(g.x, kp), _token(g.B, kp), _token(g.dt_raw, kp), w_in,
                        s_in, work_w, work_s, one, _token(g.x, k), _token(g.B, k), _token(g.C, k),
                        _token(g.dt_raw, k), y, cst, vst)
        torch.cuda.synchronize()
        assert (cst.cpu().numpy() == 0).all() and (vst.cpu().numpy() == 0).all()
        ys.append(y[:, :, 0].double().cpu().numpy())
    # rollback: commit the accepted prefix of the logged chain from the root state
    acc = np.array([3, K][:cfg.Bsz], np.int32)
    path = torch.from_numpy(np.tile(np.arange(K, dtype=np.int32), (cfg.Bsz, 1))).cuda()
    plen = torch.from_numpy(acc).cuda()
    dimsK = m.make_dims(cfg.L, cfg.Bsz, K, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.bf16)
    s_out, w_out = torch.empty_like(g.state), torch.empty_like(g.window)
    m.commit(dimsK, prm, g.parent, path, plen, g.x, g.B, g.dt_raw, g.window, g.state, w_out, s_out, cst)
    torch.cuda.synchronize()
    assert (cst.cpu().numpy() == 0).all()
    o = oracle.get()
    for l in range(cfg.L):
        for b in range(cfg.Bsz):
            u = C.unit_f64(cfg, l, b, log_inp)
            y_scan, s_scan, w_scan = o.scan(u, K, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W)
            for k in range(K):
                assert_close(ys[k][l, b], y_scan[k], "draft token %d l=%d b=%d" % (k, l, b))
            n = int(acc[b])
            _, s_pref, w_pref = o.scan(u, n, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W)
            assert_close(s_out[l, b].double().cpu().numpy(), s_pref, "rollback state l=%d b=%d" % (l, b))
            assert np.array_equal(window_f64(cfg, w_out, l, b), w_pref), "rollback window l=%d b=%d" % (l, b)


# ----------------------------------------------------------------------------
# the fused round along long accepted paths, every conv width
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_fused_round_long_paths_every_width(W):
    """The previous tree is a 16-chain whose accepted paths run 0, 1, 3, 4,
    5, 8, 15 and 16 nodes (the fused kernel spreads the path's conv over its
    four waves), the next tree a random forest; conv widths 1-4, SiLU and a
    bias on the even widths, bf16 and fp32 inputs alternating."""
    cfg = C.Config(260 + W, "long-paths", 2, 8, 16, 4, 64, 64, 1, W, W % 2 == 1, 0.5, "chain", W % 2 == 0,
                   W % 2 == 0)
    prev = C.make_inputs(cfg)
    for b, n in enumerate([0, 1, 3, 4, 5, 8, 15, 16]):
        prev.path[b, :] = -1
        prev.path[b, :n] = np.arange(n, dtype=np.int32)
        prev.path_len[b] = n
    nxt = C.make_inputs(cfg.replace(cid=cfg.cid + 500, tree="forest"), skip=NEXT_ONLY)
    log("fused round, 16-chain paths, W=%d" % W)
    step = Step(cfg, prev=prev, nxt=nxt)
    assert fused_applies(cfg)
    out = step.run()
    check(step, out, [(l, b) for l in range(cfg.L) for b in range(cfg.Bsz)])


@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_tt_round_long_paths_every_width(W):
    """The one-launch round of trees of 17-64 nodes along long accepted
    paths: the previous tree is a 64-chain whose accepted paths run 0, 1, 3,
    4, 5, 17, 63 and 64 nodes (four path positions per matrix-core product,
    the last group partly past the path), the next tree a random forest;
    conv widths 1-4, SiLU and a bias on the even widths, d_state 32 and
    128, 8 and 16 blocks per workgroup."""
    cfg = C.Config(270 + W, "tt-long-paths", 2, 8, 64, 8 if W % 2 else 16, 64, 32 if W % 2 else 128, 1, W, True,
                   0.5, "chain", W % 2 == 0, W % 2 == 0)
    assert tt_round_applies(cfg)
    prev = C.make_inputs(cfg)
    for b, n in enumerate([0, 1, 3, 4, 5, 17, 63, 64]):
        prev.path[b, :] = -1
        prev.path[b, :n] = np.arange(n, dtype=np.int32)
        prev.path_len[b] = n
    nxt = C.make_inputs(cfg.replace(cid=cfg.cid + 500, tree="forest"), skip=NEXT_ONLY)
    log("one-launch round, 64-chain paths, W=%d" % W)
    step = Step(cfg, prev=prev, nxt=nxt)
    out = step.run()
    check(step, out, [(l, b) for l in range(cfg.L) for b in range(cfg.Bsz)])


# L, Bsz, T, H, P, N, G, W, silu, bias, tree
TT_ROUND_SPECS = [
    (1, 3, 17, 8, 64, 16, 1, 4, False, False, "forest"),
    (1, 3, 32, 8, 64, 32, 1, 3, True, True, "forest"),
    (2, 2, 33, 16, 64, 64, 2, 2, False, True, "forest"),
    (1, 3, 48, 8, 128, 128, 1, 1, True, False, "forest"),       # two blocks per head
    (1, 2, 49, 16, 64, 128, 1, 4, False, False, "chain_or_star"),
    (1, 3, 64, 8, 64, 64, 1, 4, True, True, "forest"),
]


@pytest.mark.parametrize("spec", TT_ROUND_SPECS, ids=lambda s: "T%dH%dP%dN%dG%dW%d" % s[2:8])
def test_tt_round_small(spec):
    """Every tile count (17, 32, 33, 48, 49, 64 nodes), d_state 16-128, one
    and two B/C groups, all units against the oracle."""
    L, Bsz, T, H, P, N, G, W, silu, bias, tree = spec
    cfg = C.Config(280 + TT_ROUND_SPECS.index(spec), "tt-round", L, Bsz, T, H, P, N, G, W, True, 0.5, tree, silu,
                   bias)
    assert tt_round_applies(cfg)
    log("one-launch round %s" % (spec,))
    step = Step(cfg)
    check(step, step.run(), [(l, b) for l in range(L) for b in range(Bsz)])
