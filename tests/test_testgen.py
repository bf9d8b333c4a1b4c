"""The seeded input generator and the workload table (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

import testgen
from testgen import configs as C
from tests.pins import _is_bfs_labelling

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_counter_based_slices_match_full_draw():
    full = testgen.fill((1000,), 123, 7, testgen.DIST_NORMAL, 0.0, 1.0, bf16=False, nthreads=4)
    part = testgen.fill((100,), 123, 7, testgen.DIST_NORMAL, 0.0, 1.0, bf16=False, offset=437, nthreads=1)
    assert np.array_equal(full[437:537], part)
    again = testgen.fill((1000,), 123, 7, testgen.DIST_NORMAL, 0.0, 1.0, bf16=False, nthreads=1)
    assert np.array_equal(full, again)
    other = testgen.fill((1000,), 123, 8, testgen.DIST_NORMAL, 0.0, 1.0, bf16=False)
    assert not np.array_equal(full, other)


def test_distributions():
    n = 400000
    z = testgen.fill((n,), 5, 1, testgen.DIST_NORMAL, 0.0, 1.0, bf16=False).astype(np.float64)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1.0) < 0.01
    # Box-Muller tail mass beyond 3 sigma ~ 0.0027
    assert 0.0020 < np.mean(np.abs(z) > 3) < 0.0034
    u = testgen.fill((n,), 5, 2, testgen.DIST_UNIFORM, -4.0, -2.0, bf16=False).astype(np.float64)
    assert u.min() >= -4 and u.max() <= -2 and abs(u.mean() + 3) < 0.01
    a = testgen.fill((n,), 5, 3, testgen.DIST_NEG_EXP_UNIFORM, 0.0, np.log(16), bf16=False).astype(np.float64)
    assert a.max() <= -1.0 and a.min() >= -16.0
    assert abs(np.mean(np.log(-a)) - np.log(16) / 2) < 0.01


def test_bf16_rounding_matches_torch():
    f = testgen.fill((100000,), 9, 4, testgen.DIST_NORMAL, 0.0, 3.0, bf16=False)
    b = testgen.fill((100000,), 9, 4, testgen.DIST_NORMAL, 0.0, 3.0, bf16=True)
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, want)
    assert np.array_equal(testgen.f32_to_bf16_bits(f), want)
    back = testgen.bf16_bits_to_f32(b)
    assert np.array_equal(back, torch.from_numpy(f).to(torch.bfloat16).float().numpy())


def test_unit_slices_equal_full_tensors():
    cfg = C.CONFIGS[0].replace(L=2, Bsz=3, T=5)
    inp = C.make_inputs(cfg)
    for l in range(2):
        for b in range(3):
            a = C.unit_f64(cfg, l, b, inp)
            r = C.unit_f64(cfg, l, b, None)
            for k in a:
                assert np.array_equal(a[k], r[k]), k


@pytest.mark.parametrize("cid", [0, 1, 2, 3])
def test_trees_and_paths(cid):
    cfg = C.CONFIGS[cid]
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    parent, path, plen = C.make_trees(cfg, rng)
    with open(os.path.join(GOLDEN, "tree_config_specmamba.json")) as f:
        g = json.load(f)
    for b in range(cfg.Bsz):
        p = parent[b]
        assert _is_bfs_labelling(p)
        dep = C.depths(p)
        nk = np.bincount(p[p >= 0], minlength=cfg.T)
        if cfg.tree == "rand_b3_d4":
            assert nk.max() <= g["tree_config"]["max_branches"] and dep.max() <= g["tree_config"]["max_depth"]
        if cfg.tree == "spine_b23_d45":
            lo, hi = g["recommended"]["branching"]
            assert nk.max() <= hi and nk.max() >= lo
            dlo, dhi = g["recommended"]["depth"]
            assert dlo <= dep.max() <= dhi
        n = int(plen[b])
        pth = path[b, :n]
        for k, v in enumerate(pth):
            assert p[v] == (-1 if k == 0 else pth[k - 1])
        assert np.all(path[b, n:] == -1)
    if cfg.tree == "spine_b23_d45":
        lo, hi = g["recommended"]["predicted_length"]
        assert lo <= cfg.T <= hi


def test_stress_trees():
    cfg = C.CONFIGS[4]
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    parent, path, plen = C.make_trees(cfg, rng)
    assert np.array_equal(parent[0], C.chain(64))
    assert np.array_equal(parent[1], C.star(64))
    for b in range(2, cfg.Bsz):
        p = parent[b]
        assert _is_bfs_labelling(p)
        assert C.depths(p).max() <= 8
        assert np.bincount(p[p >= 0]).max() <= 4


def test_state_bf16_is_stored_as_bf16_bits():
    """With state_bf16 the root state is drawn like the fp32 state and kept
    as bfloat16 bits; the oracle's float64 view of it is exact."""
    cfg = C.Config(95, "tiny", 1, 2, 3, 2, 16, 16, 1, 4, True, 0.5, "forest", state_bf16=True)
    inp = C.make_inputs(cfg)
    assert inp.state.dtype == np.uint16 and inp.state.shape == (1, 2, 2, 16, 16)
    u = C.unit_f64(cfg, 0, 1, inp)
    as32 = u["state"].astype(np.float32)
    assert np.array_equal(as32.astype(np.float64), u["state"])
    assert not (as32.view(np.uint32) & 0xFFFF).any(), "not on the bf16 grid"
    f32 = C.make_inputs(cfg.replace(state_bf16=False)).state
    assert np.abs(u["state"] - f32[0, 1]).max() <= 2.0 ** -8 * np.abs(f32[0, 1]).max()
