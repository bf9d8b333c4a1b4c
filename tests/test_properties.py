"""Property tests of the float64 oracle (CPU): hypothesis draws the shape,
the tree, the accepted path and the inputs, and each case must satisfy the
invariants the fixed pins check on their own grids:

  * a chain tree is the plain sequential scan;
  * every node's y equals a fresh scan of its root path (SpecMamba page,
    sec. 3.2: the walk keeps verification exact);
  * committing an accepted path and then verifying the next token as a
    one-node tree equals a scan over path + token (sec. 3.1: recompute from
    the stored dt, B and x);
  * relabelling siblings in another breadth-first order permutes y alike.
"""
import numpy as np
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

import oracle  # noqa: E402
from tests.pins import rand_unit, root_path, take  # noqa: E402

SETTINGS = settings(max_examples=200, deadline=None, derandomize=True)


@pytest.fixture(scope="module")
def o():
    return oracle.get()


@st.composite
def shapes(draw):
    G = draw(st.sampled_from([1, 2]))
    H = G * draw(st.integers(1, 3))
    P = draw(st.sampled_from([1, 2, 4]))
    N = draw(st.sampled_from([1, 2, 4]))
    W = draw(st.integers(1, 4))
    silu = draw(st.booleans())
    xbc = draw(st.booleans())
    gate = draw(st.booleans())
    cb = draw(st.booleans())
    return H, P, N, G, W, silu, xbc, gate, cb


@st.composite
def trees(draw, tmax=12):
    """A breadth-first parent[] (a forest allowed): non-decreasing, each
    entry below its own index."""
    T = draw(st.integers(1, tmax))
    p = [-1]
    for i in range(1, T):
        p.append(draw(st.integers(p[-1], i - 1)))
    return np.array(p, np.int32)


def _close(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    err = np.max(np.abs(a - b) / (1e-300 + 1.0 + np.abs(b))) if a.size else 0.0
    assert err <= 1e-11, "%s: %.3g" % (what, err)


@SETTINGS
@given(shape=shapes(), T=st.integers(1, 12), seed=st.integers(0, 2**31 - 1))
def test_chain_is_scan(o, shape, T, seed):
    H, P, N, G, W, silu, xbc, gate, cb = shape
    u = rand_unit(np.random.default_rng(seed), T, H, P, N, G, W, conv_b=cb, xbc=xbc, gate=gate)
    y, stt, _ = o.verify(np.arange(-1, T - 1, dtype=np.int32), u, H, P, N, G, W, silu, xbc)
    assert stt == 0
    ys, _, _ = o.scan(u, T, H, P, N, G, W, silu, xbc)
    _close(y, ys, "chain vs scan")


@SETTINGS
@given(shape=shapes(), parent=trees(), seed=st.integers(0, 2**31 - 1))
def test_every_node_is_its_path_scan(o, shape, parent, seed):
    H, P, N, G, W, silu, xbc, gate, cb = shape
    T = len(parent)
    u = rand_unit(np.random.default_rng(seed), T, H, P, N, G, W, conv_b=cb, xbc=xbc, gate=gate)
    y, stt, _ = o.verify(parent, u, H, P, N, G, W, silu, xbc)
    assert stt == 0
    for v in range(T):
        pth = root_path(parent, v)
        ys, _, _ = o.scan(take(u, pth), len(pth), H, P, N, G, W, silu, xbc)
        _close(y[v], ys[-1], "node %d" % v)


@SETTINGS
@given(shape=shapes(), parent=trees(), leaf=st.integers(0, 63), cut=st.integers(0, 64),
       seed=st.integers(0, 2**31 - 1))
def test_commit_then_decode_is_scan(o, shape, parent, leaf, cut, seed):
    H, P, N, G, W, silu, xbc, gate, cb = shape
    T = len(parent)
    u = rand_unit(np.random.default_rng(seed), T + 1, H, P, N, G, W, conv_b=cb, xbc=xbc, gate=gate)
    uT = take(u, range(T))
    pth = root_path(parent, leaf % T)
    pth = pth[:cut % (len(pth) + 1)]  # any accepted prefix, the empty one included
    so, wo, stt = o.commit(parent, np.array(pth, np.int32), len(pth), uT, H, P, N, G, W, silu, xbc)
    assert stt == 0
    nxt = dict(take(u, [T]), state=so, window=wo)
    y1, st1, _ = o.verify(np.array([-1], np.int32), nxt, H, P, N, G, W, silu, xbc)
    assert st1 == 0
    ys, hs, ws = o.scan(take(u, pth + [T]), len(pth) + 1, H, P, N, G, W, silu, xbc)
    _close(y1[0], ys[-1], "commit then decode")
    if len(pth):
        _, hp, wp = o.scan(take(u, pth), len(pth), H, P, N, G, W, silu, xbc)
        _close(so, hp, "committed state")
        assert np.array_equal(wo, wp)


@SETTINGS
@given(shape=shapes(), parent=trees(), seed=st.integers(0, 2**31 - 1), perm_seed=st.integers(0, 1000))
def test_sibling_relabel_permutes_y(o, shape, parent, seed, perm_seed):
    """Renumber the tree by a breadth-first walk that visits each node's
    children in a random order: y follows the relabelling."""
    H, P, N, G, W, silu, xbc, gate, cb = shape
    T = len(parent)
    u = rand_unit(np.random.default_rng(seed), T, H, P, N, G, W, conv_b=cb, xbc=xbc, gate=gate)
    y, stt, _ = o.verify(parent, u, H, P, N, G, W, silu, xbc)
    assert stt == 0
    rng = np.random.default_rng(perm_seed)
    kids = {v: [c for c in range(T) if parent[c] == v] for v in range(-1, T)}
    order, frontier = [], [-1]
    while frontier:
        nxt = []
        for v in frontier:
            ch = list(kids[v])
            rng.shuffle(ch)
            order += ch
            nxt += ch
        frontier = nxt
    new_of = {old: k for k, old in enumerate(order)}
    parent2 = np.array([-1 if parent[old] < 0 else new_of[int(parent[old])] for old in order], np.int32)
    u2 = take(u, order)
    y2, st2, _ = o.verify(parent2, u2, H, P, N, G, W, silu, xbc)
    assert st2 == 0
    _close(y2, y[order], "relabelled")
