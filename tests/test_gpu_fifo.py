"""GPU parity of the explicit FIFO walk (SSM_TREE_VERIFY_FIFO): the page's
own form of verification, every child state materialised, against the
float64 oracle's literal walk; plus the fallback for trees whose live-state
peak exceeds the queue capacity.

Tolerance as for the default path: |gpu - oracle| <= 1e-5 + 1e-4 |oracle|.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mamba2_tree_verification_amd as m  # noqa: E402
import oracle  # noqa: E402
from testgen import configs as C  # noqa: E402
from tests.gpu_util import GpuCase, assert_close, check_verify, log, sample_units  # noqa: E402
from tests.test_gpu_parity import SMALL  # noqa: E402

pytestmark = pytest.mark.gpu

# States the kernel's queue holds at d_state 128 for trees of up to 25 nodes:
# the queue sits in LDS next to the per-node tables, two workgroups of 32
# channels per CU (4 slots of 16 KiB); a larger peak takes the replay
# fallback.
QUEUE_CAPACITY = 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load()


@pytest.mark.parametrize("cid,k", [(0, 1), (1, 4), (2, 4), (3, 6), (4, 4)])
def test_fifo_config_full_size(cid, k):
    cfg = C.CONFIGS[cid]
    log("fifo config %d %s" % (cid, cfg.name))
    case = GpuCase(cfg, fifo=True)
    rng = np.random.default_rng(200 + cid)
    must = [(cfg.L - 1, cfg.Bsz - 1), (0, 0)]
    if cid == 4:
        must += [(cfg.L // 2, 0), (cfg.L // 3, 1)]  # the 64-chain and the 64-star
        # the sequences whose trees exceed the queue capacity (replay fallback)
        o = oracle.get()
        over = [b for b in range(cfg.Bsz) if o.plan(case.inp.parent[b], cfg.W)[2]["peak_fifo"] > QUEUE_CAPACITY]
        assert over, "the stress workload should contain trees past the queue capacity"
        must += [(1, b) for b in over[:3]]
    units = sample_units(cfg, k, rng, must)
    y, st = case.verify()
    check_verify(case, y, st, units)


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: "L%dB%dT%dN%dP%d%s" % (s[0], s[1], s[2], s[5], s[4],
                                                                          "bf" if s[8] else "f32"))
def test_fifo_small_random(spec):
    L, Bsz, T, H, P, N, G, W, bf16, silu, bias, tree = spec
    cfg = C.Config(90 + SMALL.index(spec), "small", L, Bsz, T, H, P, N, G, W, bf16, 0.5, tree, silu, bias)
    case = GpuCase(cfg, fifo=True)
    y, st = case.verify()
    check_verify(case, y, st, [(l, b) for l in range(L) for b in range(Bsz)])


# instances the small set leaves out: float32 inputs at d_state 256 (the
# widest lane segment), 32 and 64
FIFO_F32 = [
    # L, Bsz, T, H, P, N, G, W, bf16, silu, bias, tree
    (1, 2, 24, 2, 64, 256, 1, 4, False, True, False, "forest"),
    (2, 2, 16, 4, 32, 32, 2, 3, False, False, True, "forest"),
    (1, 3, 40, 2, 64, 64, 1, 4, False, False, False, "chain_or_star"),
]


@pytest.mark.parametrize("spec", FIFO_F32, ids=lambda s: "T%dN%dP%d" % (s[2], s[5], s[4]))
def test_fifo_float32_instances(spec):
    L, Bsz, T, H, P, N, G, W, bf16, silu, bias, tree = spec
    cfg = C.Config(60 + FIFO_F32.index(spec), "small", L, Bsz, T, H, P, N, G, W, bf16, 0.5, tree, silu, bias)
    case = GpuCase(cfg, fifo=True)
    y, st = case.verify()
    check_verify(case, y, st, [(l, b) for l in range(L) for b in range(Bsz)])


def _wide_tree(n_internal, fanout):
    """Root with n_internal internal children, each with `fanout` leaves:
    every internal child is queued before the first is expanded, so the
    peak queue occupancy is n_internal."""
    par = [-1] + [0] * n_internal
    for i in range(n_internal):
        par += [1 + i] * fanout
    return np.array(par, np.int32)


@pytest.mark.parametrize("n_internal", [QUEUE_CAPACITY, QUEUE_CAPACITY + 1, 20])
def test_fifo_capacity_boundary(n_internal):
    par = _wide_tree(n_internal, 2)
    T = len(par)
    assert oracle.get().plan(par, 4)[2]["peak_fifo"] == n_internal
    cfg = C.Config(70, "wide", 2, 2, T, 2, 64, 128, 1, 4, True, 0.5, "forest")
    inp = C.make_inputs(cfg)
    inp.parent[:] = par
    case = GpuCase(cfg, inp, fifo=True)
    y, st = case.verify()
    check_verify(case, y, st, [(l, b) for l in range(cfg.L) for b in range(cfg.Bsz)])
    # and the default (root-projection) path agrees with it
    yp, _ = GpuCase(cfg, inp).verify()
    assert_close(y.double().cpu().numpy(), yp.double().cpu().numpy(), "fifo vs projection")


def test_fifo_invalid_tree_is_nan_and_isolated():
    cfg = C.Config(71, "edge", 2, 3, 12, 4, 64, 128, 1, 4, True, 0.5, "forest")
    inp = C.make_inputs(cfg)
    inp.parent[1, 4] = 7  # forward reference
    case = GpuCase(cfg, inp, fifo=True)
    y, st = case.verify()
    stn = st.cpu().numpy()
    assert stn[1] == m.E_TREE and stn[0] == 0 and stn[2] == 0
    assert torch.isnan(y[:, 1]).all()
    check_verify(case, y, st, [(l, b) for l in range(cfg.L) for b in (0, 2)])
