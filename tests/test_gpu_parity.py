"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Tolerance (the build's target): |gpu - oracle| <= 1e-5 + 1e-4 |oracle| for y
and the committed state; statuses, windows and the plan exactly.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mamba2_tree_verification_amd as m  # noqa: E402
import oracle  # noqa: E402
from testgen import configs as C  # noqa: E402
from tests.gpu_util import (GpuCase, check_commit, check_verify, log, sample_units)  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load()


# ----------------------------------------------------------------------------
# the five workloads at full size, sampled (layer, sequence) units
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("cid,k", [(0, 1), (1, 6), (2, 6), (3, 8), (4, 4)])
def test_config_full_size(cid, k):
    cfg = C.CONFIGS[cid]
    log("config %d %s: generating" % (cid, cfg.name))
    case = GpuCase(cfg)
    rng = np.random.default_rng(100 + cid)
    must = [(cfg.L - 1, cfg.Bsz - 1), (0, 0)]
    if cid == 4:
        must += [(cfg.L // 2, 0), (cfg.L // 3, 1)]  # the 64-chain and the 64-star
    units = sample_units(cfg, k, rng, must)
    log("config %d: verify on GPU" % cid)
    y, st = case.verify()
    assert not torch.isnan(y).any(), "NaN in y"
    log("config %d: oracle verify on %d units" % (cid, len(units)))
    check_verify(case, y, st, units)
    del y
    log("config %d: commit on GPU" % cid)
    s_out, w_out, st2 = case.commit()
    log("config %d: oracle commit" % cid)
    check_commit(case, s_out, w_out, st2, units)


# ----------------------------------------------------------------------------
# small random workloads covering shapes, dtypes, flags and tree families
# ----------------------------------------------------------------------------

SMALL = [
    # L, Bsz, T, H, P, N, G, W, bf16, silu, bias, tree
    (2, 3, 16, 8, 64, 128, 1, 4, True, False, False, "forest"),
    (3, 2, 5, 2, 64, 64, 1, 4, False, False, True, "forest"),
    (1, 4, 13, 4, 32, 32, 2, 3, True, True, False, "forest"),
    (2, 2, 31, 2, 128, 16, 1, 2, False, False, False, "forest"),
    (1, 3, 40, 3, 64, 256, 3, 1, True, False, True, "forest"),
    (2, 2, 64, 2, 64, 128, 1, 4, True, False, False, "chain_or_star"),
    (1, 2, 1, 8, 16, 16, 1, 4, False, True, True, "forest"),
    (2, 5, 9, 12, 16, 64, 1, 4, True, False, False, "forest"),
    (1, 2, 24, 5, 64, 128, 5, 4, True, False, False, "forest"),
    # 17..64-node trees on the matrix cores: one column group (d_state 16)
    # and heads of 16 channels (four heads per 64-channel block), silu
    (1, 3, 20, 8, 16, 16, 1, 4, True, True, False, "forest"),
    # heads of 32 channels (two heads per block), width 3, bias
    (2, 2, 50, 8, 32, 32, 2, 3, True, True, True, "forest"),
    # fp32 inputs, chain and star trees of 33 nodes, silu
    (1, 2, 33, 4, 64, 128, 1, 4, False, True, False, "chain_or_star"),
    # 17-64 nodes with 8 or 16 one-head blocks per B/C group (the role-split
    # kernel): 8 blocks; 16 blocks with chains and stars and silu; fp32
    # inputs with bias; two groups of 8 blocks
    (1, 2, 40, 8, 64, 128, 1, 4, True, False, False, "forest"),
    (1, 2, 64, 16, 64, 64, 1, 4, True, True, False, "chain_or_star"),
    (1, 2, 33, 8, 64, 64, 1, 3, False, False, True, "forest"),
    (1, 2, 24, 16, 64, 32, 2, 4, True, False, False, "forest"),
    # 40 and 24 one-head blocks per group: verify takes 40 and 24 blocks per
    # workgroup, the one-launch round 20 and 12
    (1, 2, 40, 40, 64, 64, 1, 4, True, False, False, "forest"),
    (1, 2, 20, 24, 64, 32, 1, 3, True, True, True, "chain_or_star"),
]


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: "L%dB%dT%dH%dP%dN%dG%dW%d%s%s%s" % (
    s[0], s[1], s[2], s[3], s[4], s[5], s[6], s[7], "bf" if s[8] else "f32", "S" if s[9] else "",
    "b" if s[10] else ""))
def test_small_random(spec):
    L, Bsz, T, H, P, N, G, W, bf16, silu, bias, tree = spec
    cfg = C.Config(90 + SMALL.index(spec), "small", L, Bsz, T, H, P, N, G, W, bf16, 0.5, tree, silu, bias)
    log("small %s" % (spec,))
    case = GpuCase(cfg)
    units = [(l, b) for l in range(L) for b in range(Bsz)]
    y, st = case.verify()
    check_verify(case, y, st, units)
    s_out, w_out, st2 = case.commit()
    check_commit(case, s_out, w_out, st2, units)


# ----------------------------------------------------------------------------
# bookkeeping, errors, in-place, determinism, degenerate sizes
# ----------------------------------------------------------------------------

def _small_cfg(**kw):
    base = C.Config(80, "edge", 2, 4, 12, 4, 64, 128, 1, 4, True, 0.5, "forest")
    return base.replace(**kw)


def test_plan_matches_oracle_exactly():
    rng = np.random.default_rng(7)
    trees = [C.chain(64), C.star(64), C.chain(1), np.array([-1, -1, -1, 0, 0, 2], np.int32)]
    trees += [C.random_forest(rng, int(rng.integers(1, 65))) for _ in range(40)]
    trees += [C.random_tree(rng, 16, 3, 5, spine=5) for _ in range(10)]
    o = oracle.get()
    for W in (1, 2, 3, 4):
        for par in trees:
            T = len(par)
            dims = m.make_dims(1, 1, T, 1, 64, 16, 1, W, True)
            pd = torch.from_numpy(par.astype(np.int32)).cuda()
            out = torch.full((m.PLAN_HEADER + T * m.PLAN_STRIDE,), -999, dtype=torch.int32, device="cuda")
            m.plan(dims, pd, out)
            torch.cuda.synchronize()
            g = out.cpu().numpy()
            st, plan, info = o.plan(par, W)
            assert st == 0 and g[0] == 0
            assert g[1] == info["peak_fifo"] and g[2] == info["max_depth"] and g[3] == info["n_internal"]
            assert np.array_equal(g[4:].reshape(T, 8), plan), (par.tolist(), W)


@pytest.mark.parametrize("T,P", [(12, 64), (40, 64), (40, 32)], ids=["T12", "T40", "T40P32"])
def test_invalid_trees_flagged_and_isolated(T, P):
    """Up to 16 nodes and past 16 (the 17-64-node kernel, with M shared by
    the workgroup's waves or formed per wave)."""
    cfg = _small_cfg(T=T, P=P, H=4 if P == 64 else 8, cid=80 + T + P)
    inp = C.make_inputs(cfg)
    inp.parent[1, 3] = 5          # forward reference
    inp.parent[2, 0] = 0          # first node not attached to the root state
    inp.parent[3, 5] = -2         # below -1
    inp.parent[0, 0] = -1
    case = GpuCase(cfg, inp)
    y, st = case.verify()
    stn = st.cpu().numpy()
    assert stn[0] == 0 and all(stn[b] == m.E_TREE for b in (1, 2, 3)), stn
    for b in (1, 2, 3):
        assert torch.isnan(y[:, b]).all()
    check_verify(case, y, st, [(l, 0) for l in range(cfg.L)])
    s_out, w_out, st2 = case.commit()
    check_commit(case, s_out, w_out, st2, [(l, b) for l in range(cfg.L) for b in range(cfg.Bsz)])
    assert (s_out[:, 1:4] == -777.0).all(), "failed sequences must stay unwritten"


@pytest.mark.parametrize("T", [12, 40])
def test_invalid_paths_flagged_and_untouched(T):
    cfg = _small_cfg(tree="chain_or_star", Bsz=4, T=T, cid=80 + T)
    inp = C.make_inputs(cfg)
    inp.path_len[:] = [3, 2, 3, T + 1]
    inp.path[0, :3] = [0, 1, 2]            # valid chain prefix
    inp.path[1, :2] = [1, 2]               # star: starts below the root
    inp.path[2, :3] = [0, 2, 1]            # chain: broken link
    case = GpuCase(cfg, inp)
    s_out, w_out, st = case.commit()
    stn = st.cpu().numpy()
    assert list(stn) == [0, m.E_PATH, m.E_PATH, m.E_PATH], stn
    check_commit(case, s_out, w_out, st, [(l, b) for l in range(cfg.L) for b in range(cfg.Bsz)])
    assert (s_out[:, 1:] == -777.0).all()
    # in place: failed sequences keep their input state and window
    s_in = case.g.state.clone()
    w_in = case.g.window.clone()
    s2, w2, st3 = case.commit(inplace=True, state=s_in, window=w_in)
    assert torch.equal(s2[:, 1:], case.g.state[:, 1:]) and torch.equal(w2[:, 1:], case.g.window[:, 1:])


def test_inplace_commit_equals_out_of_place():
    cfg = _small_cfg(Bsz=6)
    case = GpuCase(cfg)
    s_ref, w_ref, _ = case.commit()
    s_in, w_in = case.g.state.clone(), case.g.window.clone()
    s_out, w_out, st = case.commit(inplace=True, state=s_in, window=w_in)
    assert s_out.data_ptr() == s_in.data_ptr()
    assert torch.equal(s_out, s_ref) and torch.equal(w_out, w_ref)


def test_repeated_runs_bitwise_identical():
    cfg = _small_cfg(Bsz=3, T=16)
    case = GpuCase(cfg)
    y1, _ = case.verify()
    y2, _ = case.verify()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    s1, w1, _ = case.commit()
    s2, w2, _ = case.commit()
    assert torch.equal(s1, s2) and torch.equal(w1, w2)


def test_per_layer_calls_equal_batched_call():
    cfg = _small_cfg(L=3, Bsz=2, T=10)
    case = GpuCase(cfg)
    y_all, _ = case.verify()
    g = case.g
    for l in range(cfg.L):
        dims = m.make_dims(1, cfg.Bsz, cfg.T, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.bf16)
        prm = m.make_params(g.A[l:l + 1].contiguous(), g.D[l:l + 1].contiguous(), g.dt_bias[l:l + 1].contiguous(),
                            g.conv_w[l:l + 1].contiguous(), None)
        y = torch.empty((1, cfg.Bsz, cfg.T, cfg.d_in), dtype=torch.float32, device="cuda")
        m.verify(dims, prm, g.parent, g.x[l:l + 1].contiguous(), g.B[l:l + 1].contiguous(),
                 g.C[l:l + 1].contiguous(), g.dt_raw[l:l + 1].contiguous(), g.window[l:l + 1].contiguous(),
                 g.state[l:l + 1].contiguous(), y)
        torch.cuda.synchronize()
        assert torch.equal(y[0].view(torch.int32), y_all[l].view(torch.int32))


def test_zero_sizes():
    for kw in (dict(T=0), dict(L=0), dict(Bsz=0)):
        cfg = _small_cfg(**kw)
        case = GpuCase(cfg)
        y, st = case.verify()
        if cfg.Bsz:
            assert (st.cpu().numpy() == (0 if cfg.L else 12345)).all()
        s_out, w_out, st2 = case.commit()
        if cfg.L and cfg.Bsz:
            assert torch.equal(s_out, case.g.state) and torch.equal(w_out, case.g.window)
            assert (st2.cpu().numpy() == 0).all()


def test_commit_then_decode_matches_scan():
    """GPU commit of the accepted prefix, then a GPU verify of a 1-node tree,
    equals the oracle's plain scan over prefix + next token."""
    cfg = _small_cfg(L=2, Bsz=3, T=8, tree="chain_or_star")
    inp = C.make_inputs(cfg)
    case = GpuCase(cfg, inp)
    s_out, w_out, _ = case.commit()
    g = case.g
    nxt = C.make_inputs(cfg.replace(cid=81, T=1, tree="chain"))
    gn = GpuCase(cfg.replace(cid=81, T=1, tree="chain"), nxt)
    # next token's inputs, committed state and window, same parameters as the tree
    y = torch.empty((cfg.L, cfg.Bsz, 1, cfg.d_in), dtype=torch.float32, device="cuda")
    m.verify(gn.dims, case.prm, gn.g.parent, gn.g.x, gn.g.B, gn.g.C, gn.g.dt_raw, w_out, s_out, y)
    torch.cuda.synchronize()
    o = oracle.get()
    from tests.gpu_util import assert_close
    for l in range(cfg.L):
        for b in range(cfg.Bsz):
            u = C.unit_f64(cfg, l, b, inp)
            un = C.unit_f64(nxt.cfg, l, b, nxt)
            n = int(inp.path_len[b])
            pth = list(inp.path[b, :n])
            seq = dict(u)
            for k in ("x", "B", "C", "dt_raw"):
                seq[k] = np.concatenate([u[k][pth], un[k]], axis=0)
            ys, _, _ = o.scan(seq, n + 1, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W)
            assert_close(y[l, b, 0].double().cpu().numpy(), ys[-1], "decode after commit l=%d b=%d" % (l, b))
    del g
