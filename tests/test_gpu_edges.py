"""GPU parity at the numeric edges of the method, against the float64 oracle.

* Step sizes in both softplus tails: dt_raw + dt_bias from about -48 to 40,
  so that softplus takes its z > 20 branch (dt = z) and, far below zero,
  dt -> 0 with dA = exp(dt A) = 1 in float32.
* A root state of magnitude about 1e3.
* NaN and infinities planted in x, B, C, dt_raw, the root state and the
  conv window, each in a (layer, sequence) unit of its own.

Each runs on every kernel family: the <= 16-node verify and the fused
round, the 17-64-node matrix-core verifies (one- and two-role), the
vector-ALU verify (headdim 40, dense and deep trees), the commit, and the
explicit FIFO walk.

Where the oracle is finite the comparison is

    |gpu - oracle| <= 1e-5 + 1e-4 |oracle| + 2^-20 |.|-scale,

the elementwise band of the other parity tests widened by 16 float32 ulps
of the result's scale: the same oracle run on the absolute values of every
input (|x|, |B|, |C|, |state|, |D|, |conv weights|, window; dt and dA are
positive already), which bounds the sum of the magnitudes of the terms that
make up each output.  With steps of 20-40 and a state of 1e3 the terms of y
reach 1e3-1e5 while y itself can cancel to 0.1, and any float32 evaluation
of those terms (the fp32 state and accumulation the method specifies) is
off by a few ulps of their magnitude, not of y's; the normal workloads stay
inside the plain band.  The GPU result must be non-finite exactly where the
oracle's is (the definition: y_v depends on v's root path only, so a
non-finite input reaches exactly the outputs whose root path, conv taps or
state carry it); NaN may stand where the oracle has an infinity.  Statuses
and windows are compared exactly (windows as bits, NaN included).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mamba2_tree_verification_amd as m  # noqa: E402
import oracle  # noqa: E402
from testgen import as_f64, f32_to_bf16_bits  # noqa: E402
from testgen import configs as C  # noqa: E402
from tests.gpu_util import ATOL, RTOL, GpuCase, log  # noqa: E402
from tests.test_gpu_commit_verify import NEXT_ONLY, Step  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load()


# L, Bsz, T, H, P, N, G, W, bf16, tree   (every shape has L * Bsz >= 8 units)
SHAPES = {
    "mfma16": (2, 4, 16, 8, 64, 128, 1, 4, True, "forest"),        # <= 16 nodes, matrix cores; fused round
    "mfma16chain": (2, 4, 16, 8, 64, 128, 1, 4, True, "chain_or_star"),  # 16-chains: long sums of large steps
    "mfma12f32": (2, 4, 12, 4, 64, 64, 1, 3, False, "forest"),     # fp32 inputs
    "tt40": (2, 4, 40, 4, 64, 128, 1, 4, True, "forest"),          # 17-64 nodes, one role
    "ttws40": (2, 4, 40, 8, 64, 128, 1, 4, True, "forest"),        # 17-64 nodes, eight blocks per group
    "valu10": (2, 4, 10, 8, 40, 64, 1, 4, True, "forest"),         # headdim 40: vector ALU, dense correction
    "valu40": (2, 4, 40, 8, 40, 32, 1, 3, True, "chain_or_star"),  # headdim 40, deep trees
}


def _cfg(name, cid):
    L, Bsz, T, H, P, N, G, W, bf16, tree = SHAPES[name]
    return C.Config(cid, "edge-" + name, L, Bsz, T, H, P, N, G, W, bf16, 0.5, tree)


def _store(cfg, name, values):
    """float values in the stored form of tensor `name` (bf16 bits or float32)."""
    v = np.asarray(values, np.float32)
    return f32_to_bf16_bits(v) if C.stored_bf16(cfg, name) else v


def _put(cfg, inp, name, idx, value):
    arr = getattr(inp, name)
    arr[idx] = _store(cfg, name, np.array([value], np.float32))[0]


def dt_tails(cfg, inp, rng, dt_bias):
    """dt_raw in three regimes per (node, head): z = dt_raw + dt_bias in
    [20.5, 40] (softplus returns z), in [-48, -15] (dt below 3e-7, dA = 1 in
    float32), or the usual N(0, 1) draw."""
    shape = inp.dt_raw.shape
    regime = rng.integers(0, 3, size=shape)
    bias = dt_bias[:, None, None, :]
    hi = rng.uniform(20.5, 40.0, size=shape) - bias
    lo = rng.uniform(-48.0, -15.0, size=shape) - bias
    keep = as_f64(inp.dt_raw, C.stored_bf16(cfg, "dt_raw"))
    vals = np.where(regime == 0, hi, np.where(regime == 1, lo, keep))
    inp.dt_raw = _store(cfg, "dt_raw", vals).reshape(shape)


def big_state(cfg, inp, rng):
    inp.state = (rng.normal(scale=1e3, size=inp.state.shape)).astype(np.float32)


def _mid_node(cfg, inp, b):
    """A node with at least one descendant and, where the tree allows, a
    node that is not its descendant (the second node of the tree)."""
    par = inp.parent[b]
    T = len(par)
    kids = [v for v in range(T) if par[v] >= 0]
    return int(par[kids[len(kids) // 2]]) if kids else 0


def plant(cfg, inp):
    """One non-finite value per (layer, sequence) unit, units (0..1) x (0..3)."""
    nan, inf = float("nan"), float("inf")
    c = 3 * cfg.P + 5 if cfg.H > 3 else 5
    _put(cfg, inp, "x", (0, 0, _mid_node(cfg, inp, 0), c), nan)
    _put(cfg, inp, "x", (0, 1, _mid_node(cfg, inp, 1), c), inf)
    _put(cfg, inp, "B", (0, 2, _mid_node(cfg, inp, 2), 0, 5), nan)
    _put(cfg, inp, "C", (0, 3, _mid_node(cfg, inp, 3), 0, 7), -inf)
    _put(cfg, inp, "dt_raw", (1, 0, _mid_node(cfg, inp, 0), 1), nan)
    _put(cfg, inp, "state", (1, 1, 1, 3, 9), nan)
    _put(cfg, inp, "state", (1, 2, 0, 5, 2), inf)
    if cfg.W > 1:
        _put(cfg, inp, "window", (1, 3, cfg.W - 2, 10), nan)


SCALE_ULPS = 2.0 ** -20


def absolute(u):
    """The unit with every input replaced by its absolute value: run through
    the oracle it gives the magnitude scale of each output's terms."""
    v = dict(u)
    for k in ("x", "B", "C", "window", "state", "D", "conv_w", "conv_b", "z"):
        if v.get(k) is not None:
            v[k] = np.abs(v[k])
    return v


def assert_match(gpu, ref, what, scale=None):
    """Finite where the oracle is finite and within the tolerance there;
    non-finite exactly where the oracle is."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    band = ATOL + RTOL * np.abs(ref)
    if scale is not None:
        band = band + SCALE_ULPS * np.nan_to_num(np.asarray(scale, np.float64), nan=np.inf, posinf=np.inf)
    fin = np.isfinite(ref)
    wrong = np.isfinite(gpu) != fin
    if wrong.any():
        i = np.unravel_index(np.argmax(wrong), gpu.shape)
        raise AssertionError("%s: %d of %d differ in finiteness; first at %s gpu=%r ref=%r" %
                             (what, int(wrong.sum()), wrong.size, i, gpu[i], ref[i]))
    with np.errstate(invalid="ignore"):
        bad = fin & ~(np.abs(gpu - ref) <= band)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, np.abs(gpu - ref), -1)), gpu.shape)
        raise AssertionError("%s: %d of %d outside tolerance; worst at %s gpu=%r ref=%r" %
                             (what, int(bad.sum()), bad.size, i, gpu[i], ref[i]))


def _window_bits_equal(cfg, w_gpu, w_ref):
    g = w_gpu.float().cpu().numpy().astype(np.float64)
    return np.array_equal(np.isnan(g), np.isnan(w_ref)) and np.array_equal(np.nan_to_num(g), np.nan_to_num(w_ref))


def scales(cfg, inp, l, b, nxt=None):
    """Magnitude scales of a unit: (verify y, committed state, next tree's y)."""
    o = oracle.get()
    a = (cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.silu, cfg.xbc)
    ua = absolute(C.unit_f64(cfg, l, b, inp))
    y_s, _, _ = o.verify(inp.parent[b], ua, *a)
    n = int(inp.path_len[b])
    s_s, w_s, _ = o.commit(inp.parent[b], inp.path[b, :n], n, ua, *a)
    yn_s = None
    if nxt is not None:
        shp = C.unit_shapes(cfg)
        un = dict(ua, state=s_s, window=w_s)
        for k in ("x", "B", "C", "dt_raw"):
            un[k] = as_f64(getattr(nxt, k)[l, b], cfg.bf16).reshape(shp[k])
        un = absolute(un)  # (dt_raw kept: the step sizes are positive already)
        yn_s, _, _ = o.verify(nxt.parent[b], un, *a)
    return y_s, s_s, yn_s


def run_verify(cfg, inp, fifo=False):
    case = GpuCase(cfg, inp=inp, fifo=fifo)
    units = [(l, b) for l in range(cfg.L) for b in range(cfg.Bsz)]
    sc = {lb: scales(cfg, inp, *lb) for lb in units}
    y, st = case.verify()
    ref = case.oracle_verify(units)
    stn = st.cpu().numpy()
    for (l, b), (yr, rc, _) in ref.items():
        assert stn[b] == rc == 0, ("status", b, stn[b], rc)
        assert_match(y[l, b].double().cpu().numpy(), yr, "%s y[l=%d,b=%d]" % (cfg.name, l, b), sc[l, b][0])
    return case, units, sc


def run_verify_commit(cfg, inp):
    case, units, sc = run_verify(cfg, inp)
    s_out, w_out, st2 = case.commit()
    ref = case.oracle_commit(units)
    stn = st2.cpu().numpy()
    for (l, b), (sr, wr, rc) in ref.items():
        assert stn[b] == rc == 0, ("commit status", b, stn[b], rc)
        assert_match(s_out[l, b].double().cpu().numpy(), sr, "%s state[l=%d,b=%d]" % (cfg.name, l, b),
                     sc[l, b][1])
        if cfg.W > 1:
            assert _window_bits_equal(cfg, w_out[l, b], wr), "window l=%d b=%d" % (l, b)


def run_round(cfg, prev, nxt):
    step = Step(cfg, prev=prev, nxt=nxt)
    s_out, w_out, y, cst, vst = step.run()
    units = [(l, b) for l in range(cfg.L) for b in range(cfg.Bsz)]
    sc = {lb: scales(cfg, prev, *lb, nxt=nxt) for lb in units}
    ref = step.oracle(units)
    cs, vs = cst.cpu().numpy(), vst.cpu().numpy()
    for (l, b), (so, wo, rc, yr, rv) in ref.items():
        assert cs[b] == rc == 0 and vs[b] == rv == 0, ("status", b, cs[b], vs[b])
        assert_match(s_out[l, b].double().cpu().numpy(), so, "%s round state[l=%d,b=%d]" % (cfg.name, l, b),
                     sc[l, b][1])
        if cfg.W > 1:
            assert _window_bits_equal(cfg, w_out[l, b], wo), "round window l=%d b=%d" % (l, b)
        assert_match(y[l, b].double().cpu().numpy(), yr, "%s round y[l=%d,b=%d]" % (cfg.name, l, b), sc[l, b][2])


CASES = ["dt_tails", "big_state", "nonfinite"]


def _inputs(name, case, cid):
    cfg = _cfg(name, cid)
    rng = np.random.default_rng(cid)
    prev = C.make_inputs(cfg)
    nxt = C.make_inputs(cfg.replace(cid=cid + 500), skip=NEXT_ONLY)
    if case == "dt_tails":
        dt_tails(cfg, prev, rng, prev.dt_bias)
        dt_tails(cfg, nxt, rng, prev.dt_bias)
    elif case == "big_state":
        big_state(cfg, prev, rng)
    else:
        plant(cfg, prev)
        # the next tree gets non-finite node inputs of its own in the same units
        nan = float("nan")
        _put(cfg, nxt, "x", (1, 1, _mid_node(cfg, nxt, 1), 2), nan)
        _put(cfg, nxt, "B", (1, 2, _mid_node(cfg, nxt, 2), 0, 1), float("inf"))
    return cfg, prev, nxt


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("name", list(SHAPES))
def test_edges_verify_commit(name, case):
    cid = 700 + 10 * list(SHAPES).index(name) + CASES.index(case)
    cfg, prev, _ = _inputs(name, case, cid)
    log("edges verify+commit %s %s" % (name, case))
    run_verify_commit(cfg, prev)


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("name", list(SHAPES))
def test_edges_round(name, case):
    cid = 700 + 10 * list(SHAPES).index(name) + CASES.index(case)
    cfg, prev, nxt = _inputs(name, case, cid)
    log("edges round %s %s" % (name, case))
    run_round(cfg, prev, nxt)


# the explicit FIFO walk (SSM_TREE_VERIFY_FIFO) at the same edges: trees of
# 16 nodes (queue in LDS) and 40 nodes (queue, or the replay fallback), and
# deep chains and stars
FIFO_SHAPES = ["mfma16", "tt40", "valu40"]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("name", FIFO_SHAPES)
def test_edges_fifo_verify(name, case):
    cid = 700 + 10 * list(SHAPES).index(name) + CASES.index(case)
    cfg, prev, _ = _inputs(name, case, cid)
    log("edges fifo verify %s %s" % (name, case))
    run_verify(cfg, prev, fifo=True)
