"""GPU parity of the Mamba2-convention options against the float64 oracle
with the same options: the causal conv over x, B and C (SSM_TREE_CONV_XBC:
in_proj's xBC passes conv1d as a whole) and the output gate y * silu(z)
(LightMamba part, "why Mamba is hard to accelerate": Y is multiplied
elementwise with Z).

ssm_tree_commit takes the xBC conv for every shape; ssm_tree_verify takes
both options on trees of 1-16 nodes (the fused round's kernel with nothing
to commit) and of 17-64 nodes (the options' instantiation of the 17-64-node
matrix-core kernel), with a headdim that is a multiple of 16;
ssm_tree_commit_verify fuses them up to 16 nodes and runs the two calls
past that.  Every other combination must be refused on the host with
SSM_TREE_E_DIMS before anything is enqueued.  Tolerance as elsewhere:
|gpu - oracle| <= 1e-5 + 1e-4 |oracle|; windows and statuses exactly.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mamba2_tree_verification_amd as m  # noqa: E402
import oracle  # noqa: E402
from testgen import configs as C  # noqa: E402
from testgen.device import upload  # noqa: E402
from tests.gpu_util import (GpuCase, assert_close, check_commit, check_verify, log, sample_units,  # noqa: E402
                            window_f64)
from tests.test_gpu_commit_verify import Step, check  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load()


def _cfg(cid, **kw):
    base = C.Config(cid, "options", 2, 4, 12, 4, 64, 128, 1, 4, True, 0.5, "forest", True, False, True, True)
    return base.replace(**kw)


# ----------------------------------------------------------------------------
# ssm_tree_commit with the xBC conv (any supported shape)
# ----------------------------------------------------------------------------

COMMIT_SPECS = [  # T, H, P, N, G, W, bf16, silu, conv_b, tree
    (12, 4, 64, 128, 1, 4, True, True, False, "forest"),
    (40, 2, 64, 64, 2, 3, False, False, True, "forest"),
    (64, 2, 64, 128, 1, 4, True, True, True, "chain_or_star"),
    (9, 8, 16, 256, 1, 2, True, False, False, "forest"),
    (5, 2, 32, 16, 1, 1, False, True, False, "forest"),
    (16, 4, 48, 32, 1, 4, True, True, True, "forest"),
]


@pytest.mark.parametrize("inplace", [False, True], ids=["out", "inplace"])
@pytest.mark.parametrize("spec", COMMIT_SPECS, ids=lambda s: "T%dH%dP%dN%dG%dW%d%s" % (s[:6] + ("bf" if s[6] else "f32",)))
def test_commit_xbc(spec, inplace):
    T, H, P, N, G, W, bf16, silu, cb, tree = spec
    cfg = C.Config(150 + COMMIT_SPECS.index(spec), "xbc-commit", 2, 3, T, H, P, N, G, W, bf16, 0.5, tree, silu, cb,
                   True, False)
    log("commit xbc %s %s" % (spec, "in place" if inplace else "out of place"))
    case = GpuCase(cfg)
    s_in, w_in = case.g.state.clone(), case.g.window.clone()
    s_out, w_out, st = case.commit(inplace=inplace, state=s_in, window=w_in)
    check_commit(case, s_out, w_out, st, [(l, b) for l in range(cfg.L) for b in range(cfg.Bsz)])


def test_commit_xbc_failed_paths_untouched():
    cfg = _cfg(160, gate=False, Bsz=3)
    inp = C.make_inputs(cfg)
    inp.path_len[1] = cfg.T + 1
    inp.parent[2, 3] = 9
    case = GpuCase(cfg, inp)
    s_out, w_out, st = case.commit()
    assert list(st.cpu().numpy()) == [0, m.E_PATH, m.E_TREE]
    assert (s_out[:, 1:] == -777.0).all() and (w_out[:, 1:].float() == 0).all()
    check_commit(case, s_out, w_out, st, [(l, 0) for l in range(cfg.L)])


# ----------------------------------------------------------------------------
# the fused round with the options
# ----------------------------------------------------------------------------

ROUND_SPECS = [  # T, H, P, N, G, W, bf16, silu, conv_b, xbc, gate
    (12, 4, 64, 128, 1, 4, True, True, False, True, True),
    (16, 8, 64, 128, 1, 4, True, True, True, True, False),
    (16, 8, 64, 128, 1, 4, True, False, False, False, True),
    (7, 4, 32, 64, 2, 3, False, True, True, True, True),
    (1, 8, 16, 16, 1, 2, True, False, False, True, True),
    (13, 2, 128, 256, 1, 4, True, True, False, True, True),
    (10, 6, 32, 32, 3, 1, False, False, True, True, True),
    # 17-64 nodes: verify on the options' instantiation of the 17-64-node
    # kernel (the round as commit + verify)
    (40, 4, 64, 128, 1, 4, True, True, False, True, True),
    (64, 2, 64, 128, 1, 4, True, True, True, True, False),
    (24, 8, 32, 64, 2, 3, False, True, True, True, True),
    (33, 4, 16, 32, 1, 4, True, False, False, False, True),
    (20, 2, 128, 256, 1, 2, True, True, False, True, True),
    (50, 6, 32, 16, 3, 1, True, False, True, True, True),
]


@pytest.mark.parametrize("inplace", [False, True], ids=["out", "inplace"])
@pytest.mark.parametrize("spec", ROUND_SPECS, ids=lambda s: "T%dH%dP%dN%dG%dW%d%s%s%s" % (
    s[:6] + ("bf" if s[6] else "f32", "X" if s[9] else "", "Z" if s[10] else "")))
def test_round_options(spec, inplace):
    T, H, P, N, G, W, bf16, silu, cb, xbc, gate = spec
    cfg = C.Config(170 + ROUND_SPECS.index(spec), "opt-round", 2, 4, T, H, P, N, G, W, bf16, 0.5, "forest", silu,
                   cb, xbc, gate)
    log("round options %s %s" % (spec, "in place" if inplace else "out of place"))
    step = Step(cfg)
    if inplace:
        s_in, w_in = step.gp.state.clone(), step.gp.window.clone()
        out = step.run(inplace=True, state=s_in, window=w_in)
    else:
        out = step.run()
    check(step, out, [(l, b) for l in range(cfg.L) for b in range(cfg.Bsz)])


@pytest.mark.parametrize("spec", ROUND_SPECS, ids=lambda s: "T%dH%dP%dN%dG%dW%d%s%s%s" % (
    s[:6] + ("bf" if s[6] else "f32", "X" if s[9] else "", "Z" if s[10] else "")))
def test_verify_options(spec):
    """ssm_tree_verify alone with the options (the fused kernel with nothing
    to commit): y against the oracle's verify, state and window untouched."""
    T, H, P, N, G, W, bf16, silu, cb, xbc, gate = spec
    cfg = C.Config(200 + ROUND_SPECS.index(spec), "opt-verify", 2, 4, T, H, P, N, G, W, bf16, 0.5, "forest", silu,
                   cb, xbc, gate)
    log("verify options %s" % (spec,))
    inp = C.make_inputs(cfg)
    inp.parent[3, min(2, T - 1)] = 5 if T > 2 else -2  # one invalid tree
    case = GpuCase(cfg, inp)
    s0, w0 = case.g.state.clone(), case.g.window.clone()
    y, st = case.verify()
    assert torch.equal(case.g.state, s0) and torch.equal(case.g.window, w0)
    assert st.cpu().numpy()[3] == m.E_TREE
    check_verify(case, y, st, [(l, b) for l in range(cfg.L) for b in range(cfg.Bsz)])


def test_verify_options_full_size():
    cfg = C.CONFIGS[3].replace(cid=210, silu=True, xbc=True, gate=True)
    case = GpuCase(cfg)
    y, st = case.verify()
    assert not torch.isnan(y).any()
    units = sample_units(cfg, 6, np.random.default_rng(210), [(0, 0), (cfg.L - 1, cfg.Bsz - 1)])
    check_verify(case, y, st, units)


def test_round_options_full_size():
    """The 2.7B batch-16 tree-16 workload with both options (Mamba2
    convention: SiLU over the xBC conv, gate), sampled units."""
    cfg = C.CONFIGS[3].replace(cid=180, silu=True, xbc=True, gate=True)
    step = Step(cfg)
    out = step.run(inplace=True, state=step.gp.state.clone(), window=step.gp.window.clone())
    assert not torch.isnan(out[2]).any()
    units = sample_units(cfg, 6, np.random.default_rng(180), [(0, 0), (cfg.L - 1, cfg.Bsz - 1)])
    check(step, out, units)


def test_options_stress_full_size():
    """The stress workload (64 layers, batch 64, trees of 64 nodes: chains,
    stars, random depth <= 8) with SiLU over the xBC conv and the gate:
    verify alone, then the round (commit + verify), on sampled units
    including the 64-chain and the 64-star."""
    cfg = C.CONFIGS[4].replace(cid=220, silu=True, xbc=True, gate=True)
    log("options stress: generating")
    step = Step(cfg)
    must = [(0, 0), (cfg.L - 1, cfg.Bsz - 1), (cfg.L // 2, 0), (cfg.L // 3, 1)]
    units = sample_units(cfg, 4, np.random.default_rng(220), must)
    log("options stress: round on GPU")
    out = step.run(inplace=True, state=step.gp.state.clone(), window=step.gp.window.clone())
    assert not torch.isnan(out[2]).any()
    log("options stress: oracle on %d units" % len(units))
    check(step, out, units)


def test_round_options_failures():
    cfg = _cfg(181, Bsz=5)
    prev = C.make_inputs(cfg)
    prev.parent[1, 3] = 7
    prev.path_len[2] = cfg.T + 1
    step = Step(cfg, prev=prev)
    step.nxt.parent[3, 2] = -3
    step.gn.parent.copy_(torch.from_numpy(step.nxt.parent))
    out = step.run()
    cs, vs = out[3].cpu().numpy(), out[4].cpu().numpy()
    assert list(cs[:3]) == [0, m.E_TREE, m.E_PATH] and vs[3] == m.E_TREE
    check(step, out, [(l, b) for l in range(cfg.L) for b in range(cfg.Bsz)])


def test_draft_decode_with_options():
    """Draft tokens as one-node rounds with the xBC conv, SiLU and the gate,
    then a rollback commit on the chain, against the oracle's scan."""
    K = 6
    cfg = C.Config(182, "draft-opt", 2, 2, K, 8, 64, 128, 1, 4, True, 0.5, "chain", True, False, True, True)
    log_inp = C.make_inputs(cfg)
    g = upload(log_inp)
    dims1 = m.make_dims(cfg.L, cfg.Bsz, 1, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.bf16, cfg.silu, xbc=True)
    prm = m.make_params(g.A, g.D, g.dt_bias, g.conv_w, None)
    one = torch.full((cfg.Bsz, 1), -1, dtype=torch.int32, device="cuda")
    path0 = torch.zeros((cfg.Bsz, 1), dtype=torch.int32, device="cuda")
    ws, ww = torch.empty_like(g.state), torch.empty_like(g.window)
    cst = torch.empty((cfg.Bsz,), dtype=torch.int32, device="cuda")
    vst = torch.empty_like(cst)

    def tok(t, k):
        return t[:, :, k:k + 1].contiguous()

    ys = []
    for k in range(K):
        plen = torch.full((cfg.Bsz,), 1 if k else 0, dtype=torch.int32, device="cuda")
        kp = max(k - 1, 0)
        y = torch.empty((cfg.L, cfg.Bsz, 1, cfg.d_in), dtype=torch.float32, device="cuda")
        s_in, w_in = (g.state, g.window) if k == 0 else (ws, ww)
        m.commit_verify(dims1, prm, one, path0, plen, tok(g.x, kp), tok(g.B, kp), tok(g.dt_raw, kp), w_in, s_in,
                        ww, ws, one, tok(g.x, k), tok(g.B, k), tok(g.C, k), tok(g.dt_raw, k), y, cst, vst,
                        C_prev=tok(g.C, kp), z=tok(g.z, k))
        torch.cuda.synchronize()
        assert (cst.cpu().numpy() == 0).all() and (vst.cpu().numpy() == 0).all()
        ys.append(y[:, :, 0].double().cpu().numpy())
    acc = np.array([2, K], np.int32)
    path = torch.from_numpy(np.tile(np.arange(K, dtype=np.int32), (cfg.Bsz, 1))).cuda()
    dimsK = m.make_dims(cfg.L, cfg.Bsz, K, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.bf16, cfg.silu, xbc=True)
    s_out, w_out = torch.empty_like(g.state), torch.empty_like(g.window)
    m.commit(dimsK, prm, g.parent, path, torch.from_numpy(acc).cuda(), g.x, g.B, g.dt_raw, g.window, g.state, w_out,
             s_out, cst, C=g.C)
    torch.cuda.synchronize()
    o = oracle.get()
    for l in range(cfg.L):
        for b in range(cfg.Bsz):
            u = C.unit_f64(cfg, l, b, log_inp)
            y_scan, _, _ = o.scan(u, K, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, True, True)
            for k in range(K):
                assert_close(ys[k][l, b], y_scan[k], "draft token %d l=%d b=%d" % (k, l, b))
            n = int(acc[b])
            _, s_pref, w_pref = o.scan(u, n, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, True, True)
            assert_close(s_out[l, b].double().cpu().numpy(), s_pref, "rollback state l=%d b=%d" % (l, b))
            assert np.array_equal(window_f64(cfg, w_out, l, b), w_pref)


# ----------------------------------------------------------------------------
# combinations no kernel takes are refused before anything runs
# ----------------------------------------------------------------------------

def test_unsupported_option_combinations_refused():
    # verify alone on shapes no kernel takes with the options (headdim not a
    # multiple of 16; fp32 inputs with 64 nodes and d_state 128, whose
    # float32 B, C and raw rows exceed the LDS), and with the FIFO walk:
    # refused, y untouched
    for kw in (dict(P=40, H=8), dict(T=64, bf16=False)):
        cfg = _cfg(190, **kw)
        case = GpuCase(cfg)
        y = torch.full((cfg.L, cfg.Bsz, cfg.T, cfg.d_in), 5.0, device="cuda")
        with pytest.raises(m.SsmTreeError) as e:
            case.verify(y=y)
        assert e.value.code == m.E_DIMS and (y == 5.0).all()
    cfg = _cfg(192)
    case = GpuCase(cfg, fifo=True)
    with pytest.raises(m.SsmTreeError) as e:
        case.verify()
    assert e.value.code == m.E_DIMS
    # the round on a shape it does not fuse (T > 16): the two calls would need
    # verify to take the options, which it does not here; nothing may run,
    # the state stays
    cfg = _cfg(191, T=64, bf16=False)
    step = Step(cfg)
    s_in = step.gp.state.clone()
    with pytest.raises(m.SsmTreeError) as e:
        step.run(inplace=True, state=s_in, window=step.gp.window.clone())
    assert e.value.code == m.E_DIMS
    assert torch.equal(s_in, step.gp.state)


# ----------------------------------------------------------------------------
# the xBC conv on seeded random shapes of 1-16 nodes (the fused round and
# verify, whose convolved B/C rows and C . B table come from the workspace)
# ----------------------------------------------------------------------------

def _random_xbc_shapes(n, seed):
    """(T, H, P, N, G, W, bf16, silu, conv_b, gate): headdims that are
    multiples of 16, H*P/G a multiple of 64 (every other draw with the most
    groups the heads allow), every d_state, conv widths 1-4, both input
    types and every option combination."""
    rng = np.random.default_rng(seed)
    hp = [(4, 16), (2, 32), (4, 48), (1, 64), (2, 64), (1, 128), (8, 16), (6, 32), (4, 32)]
    hp_groups = [(8, 16), (6, 32), (4, 32), (2, 64), (4, 64)]  # head shapes that allow G > 1
    out = []
    while len(out) < n:
        pick = hp_groups if len(out) % 2 else hp
        H, P = pick[int(rng.integers(len(pick)))]
        gs = [g for g in (1, 2, 3, 4, 6, 8) if H % g == 0 and (H * P // g) % 64 == 0]
        G = int(gs[-1]) if len(out) % 2 else int(rng.choice(gs))  # every other draw: the most groups
        N = int(rng.choice([16, 32, 64, 128, 256]))
        T = int(rng.integers(1, 17))
        W = int(rng.integers(1, 5))
        bf16, silu, cb, gate = (bool(rng.integers(2)) for _ in range(4))
        out.append((T, H, P, N, G, W, bf16, silu, cb, gate))
    return out


RANDOM_XBC = _random_xbc_shapes(12, 2026)


@pytest.mark.parametrize("k", range(len(RANDOM_XBC)), ids=lambda k: "T%dH%dP%dN%dG%dW%d" % RANDOM_XBC[k][:6])
def test_xbc_random_shapes(k):
    """The round and verify alone with the xBC conv against the oracle on
    every (layer, sequence) unit."""
    T, H, P, N, G, W, bf16, silu, cb, gate = RANDOM_XBC[k]
    cfg = C.Config(950 + k, "xbc-random", 2, 3, T, H, P, N, G, W, bf16, 0.5, "forest", silu, cb, True, gate)
    log("random xBC shape %d: %s" % (k, RANDOM_XBC[k]))
    units = [(l, b) for l in range(cfg.L) for b in range(cfg.Bsz)]
    step = Step(cfg)
    check(step, step.run(), units)
    case = GpuCase(cfg)
    y, st = case.verify()
    check_verify(case, y, st, units)
