"""Pins of the float64 oracle against facts fixed outside the oracle.

Each pin takes a loaded oracle (the real one, or a build with one planted
mistake) and raises AssertionError when the oracle disagrees with:

  * a textbook special case: a chain tree is a plain sequential scan;
  * the pages' accuracy claim (SpecMamba page, sec. 3.2: the FIFO walk keeps
    verification exact): every node equals a fresh scan of its root path;
  * brute force over every BFS-ordered forest of up to 8 nodes;
  * an independently written closed form (cumulative log-decays, no
    recurrence, numpy's correlate for the conv);
  * library routines: numpy's logaddexp for softplus, scipy's lfilter for
    the first-order recurrence, numpy's correlate for the causal conv;
  * special cases with hand-derived results, and the hand-worked golden
    example in tests/golden/hand_tree3.json;
  * an independent BFS definition of valid parent[] arrays and of the plan.
"""
from __future__ import annotations

import itertools
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# inputs
# ----------------------------------------------------------------------------

def rand_unit(rng, T, H, P, N, G, W, state_std=0.5, conv_b=False, S=None, xbc=False, gate=False):
    """Random unit; with xbc the conv (window, weights, bias) spans x, B and
    C channels, with gate it carries z."""
    d = H * P
    ch = d + (2 * G * N if xbc else 0)
    n = T if S is None else S
    u = dict(
        x=rng.normal(size=(n, d)), B=rng.normal(size=(n, G, N)), C=rng.normal(size=(n, G, N)),
        dt_raw=rng.normal(size=(n, H)), window=rng.normal(size=(W - 1, ch)),
        state=rng.normal(scale=state_std, size=(H, P, N)), A=-np.exp(rng.uniform(0, np.log(16), size=H)),
        D=rng.normal(size=H), dt_bias=rng.uniform(-4, -2, size=H), conv_w=rng.normal(scale=0.5, size=(ch, W)),
    )
    u["conv_b"] = rng.normal(size=ch) if conv_b else None
    u["z"] = rng.normal(scale=2.0, size=(n, d)) if gate else None
    return u


def take(u, idx):
    """Token-indexed unit made of the nodes idx (for scans along a path)."""
    v = dict(u)
    for k in ("x", "B", "C", "dt_raw", "z"):
        if u.get(k) is None:
            continue
        v[k] = np.ascontiguousarray(u[k][list(idx)]) if len(idx) else u[k][:0].copy()
    return v


def all_bfs_forests(T):
    """Every non-decreasing parent[] with parent[0] = -1 and parent[i] < i."""
    if T == 0:
        yield np.zeros(0, np.int32)
        return

    def rec(prefix):
        i = len(prefix)
        if i == T:
            yield np.array(prefix, np.int32)
            return
        for p in range(prefix[-1], i):
            yield from rec(prefix + [p])

    yield from rec([-1])


def root_path(parent, v):
    out = []
    while v >= 0:
        out.append(int(v))
        v = int(parent[v])
    return out[::-1]


def close(a, b, tol=1e-10, what=""):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.abs(a - b) / (1.0 + np.abs(b))
    assert np.all(np.isfinite(err)) and err.max(initial=0.0) <= tol, (what, float(err.max(initial=0.0)))


# ----------------------------------------------------------------------------
# independent closed form
# ----------------------------------------------------------------------------

def closed_form_node(u, parent, v, H, P, N, G, W, silu=False, xbc=False):
    """y_v from cumulative log-decays along v's root path; no recurrence.

    With s_t = sum_{k<=t} dt_k A along the path (u_0 .. u_{m-1} = v):
      y_v = e^{s_{m-1}} C_v.h0 + sum_t e^{s_{m-1} - s_t} dt_t x~_t (C_v.B_t) + D x~_v
    and x~ the causal conv (numpy.correlate) over (window rows, path x rows);
    with xbc, B and C are the same conv of their own channels.  A gate input
    z multiplies the result by z / (1 + e^-z).
    """
    path = root_path(parent, v)
    m = len(path)
    d, gn = H * P, G * N
    ch = d + (2 * gn if xbc else 0)
    raw = np.concatenate([u["x"][path], u["B"][path].reshape(m, gn), u["C"][path].reshape(m, gn)], axis=1)[:, :ch]
    seq = np.concatenate([u["window"].reshape(W - 1, ch), raw], axis=0)  # [(W-1)+m][ch]
    conv = np.empty((m, ch))
    for c in range(ch):
        col = np.correlate(seq[:, c], u["conv_w"][c], mode="valid")  # sum_k w[k] seq[t+k]
        conv[:, c] = col + (u["conv_b"][c] if u.get("conv_b") is not None else 0.0)
    if silu:
        conv = conv / (1.0 + np.exp(-conv))
    xt = conv[:, :d]
    Bp = conv[:, d:d + gn].reshape(m, G, N) if xbc else u["B"][path]
    Cp = conv[:, d + gn:].reshape(m, G, N) if xbc else u["C"][path]
    hpg = H // G
    y = np.empty(d)
    for h in range(H):
        g = h // hpg
        dt = np.logaddexp(0.0, u["dt_raw"][path, h] + u["dt_bias"][h])
        s = np.cumsum(dt * u["A"][h])
        Cv = Cp[-1, g]
        for p in range(P):
            c = h * P + p
            tot = np.exp(s[-1]) * float(Cv @ u["state"][h, p])
            for t in range(m):
                tot += np.exp(s[-1] - s[t]) * dt[t] * xt[t, c] * float(Cv @ Bp[t, g])
            y[c] = tot + u["D"][h] * xt[-1, c]
    if u.get("z") is not None:
        z = u["z"][v]
        y = y * z / (1.0 + np.exp(-z))
    return y


# ----------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------

SHAPES = [  # (H, P, N, G, W, silu, conv_b)
    (3, 2, 5, 1, 4, False, False),
    (4, 3, 4, 2, 3, False, True),
    (2, 2, 3, 1, 2, True, False),
    (2, 1, 2, 2, 1, False, False),
]

# the Mamba2-convention options: (H, P, N, G, W, silu, conv_b, xbc, gate)
SHAPES_X = [
    (3, 2, 5, 1, 4, True, True, True, True),
    (4, 3, 4, 2, 3, False, False, True, False),
    (2, 2, 3, 1, 2, True, False, False, True),
    (2, 1, 2, 2, 1, False, True, True, True),
]


def all_shapes():
    """(H, P, N, G, W, silu, conv_b, xbc, gate) for the plain and the option shapes."""
    return [s + (False, False) for s in SHAPES] + SHAPES_X


def pin_chain_is_scan(o, seed=1):
    rng = np.random.default_rng(seed)
    for (H, P, N, G, W, silu, cb, xbc, gate) in all_shapes():
        T = 7
        u = rand_unit(rng, T, H, P, N, G, W, conv_b=cb, xbc=xbc, gate=gate)
        parent = np.arange(-1, T - 1, dtype=np.int32)
        y, st, _ = o.verify(parent, u, H, P, N, G, W, silu, xbc)
        assert st == 0
        ys, _, _ = o.scan(u, T, H, P, N, G, W, silu, xbc)
        close(y, ys, 1e-12, "chain vs scan %s" % ((H, P, N, G, W, silu, cb, xbc, gate),))


def pin_every_node_is_its_path_scan(o, seed=2, trees=6, T=10):
    rng = np.random.default_rng(seed)
    shapes = all_shapes()
    for (H, P, N, G, W, silu, cb, xbc, gate) in shapes[:2] + shapes[len(SHAPES):len(SHAPES) + 2]:
        for _ in range(trees):
            parent = _rand_parent(rng, T)
            u = rand_unit(rng, T, H, P, N, G, W, conv_b=cb, xbc=xbc, gate=gate)
            y, st, _ = o.verify(parent, u, H, P, N, G, W, silu, xbc)
            assert st == 0
            for v in range(T):
                pth = root_path(parent, v)
                ys, _, _ = o.scan(take(u, pth), len(pth), H, P, N, G, W, silu, xbc)
                close(y[v], ys[-1], 1e-12, "node %d path scan" % v)


def _rand_parent(rng, T):
    """Random BFS parent[] (possibly a forest) drawn uniformly by steps."""
    p = [-1]
    for i in range(1, T):
        p.append(int(rng.integers(p[-1], i)))
    return np.array(p, np.int32)


CATALAN = [1, 1, 2, 5, 14, 42, 132, 429, 1430]


def pin_bruteforce_forests(o, tmax=8, seed=3, tmax_options=6):
    """Every BFS forest up to tmax nodes (up to tmax_options with the xbc
    conv and the gate): every node's y equals the scan of its root path,
    and committing that path equals the scan's state and window."""
    rng = np.random.default_rng(seed)
    H, P, N, G, W = 1, 2, 2, 1, 3
    for opts in (False, True):
        for T in range(0, (tmax_options if opts else tmax) + 1):
            forests = list(all_bfs_forests(T))
            assert len(forests) == CATALAN[T], (T, len(forests))
            u = rand_unit(rng, T, H, P, N, G, W, xbc=opts, gate=opts)
            # scans of every root path that occurs in any forest of this size
            for parent in forests:
                assert o.validate_tree(parent) == 0
                y, st, _ = o.verify(parent, u, H, P, N, G, W, opts, opts)
                assert st == 0
                for v in range(T):
                    pth = root_path(parent, v)
                    ys, hs, ws = o.scan(take(u, pth), len(pth), H, P, N, G, W, opts, opts)
                    close(y[v], ys[-1], 1e-12, "forest %s node %d" % (parent.tolist(), v))
                    so, wo, cst = o.commit(parent, np.array(pth, np.int32), len(pth), u, H, P, N, G, W, opts, opts)
                    assert cst == 0
                    close(so, hs, 1e-12, "commit state")
                    assert np.array_equal(wo, ws), "commit window"


def pin_closed_form(o, seed=4):
    rng = np.random.default_rng(seed)
    for (H, P, N, G, W, silu, cb, xbc, gate) in all_shapes():
        T = 9
        parent = _rand_parent(rng, T)
        u = rand_unit(rng, T, H, P, N, G, W, conv_b=cb, xbc=xbc, gate=gate)
        y, st, _ = o.verify(parent, u, H, P, N, G, W, silu, xbc)
        assert st == 0
        for v in range(T):
            close(y[v], closed_form_node(u, parent, v, H, P, N, G, W, silu, xbc), 1e-10, "closed form node %d" % v)


def pin_softplus_library(o):
    """One node, zero root state, unit C.B, no D: y = softplus(z) * x~."""
    H, P, N, G, W = 1, 1, 1, 1, 1
    zs = np.array([-30.0, -5.0, -1.0, 0.0, 0.7, 3.0, 15.0, 19.5, 20.5, 35.0])
    for z in zs:
        u = dict(x=np.array([[1.0]]), B=np.array([[[1.0]]]), C=np.array([[[1.0]]]), dt_raw=np.array([[z]]),
                 window=np.zeros((0, 1)), state=np.zeros((1, 1, 1)), A=np.array([-1.0]), D=np.array([0.0]),
                 dt_bias=np.array([0.0]), conv_w=np.array([[1.0]]), conv_b=None)
        y, st, _ = o.verify(np.array([-1], np.int32), u, H, P, N, G, W)
        want = np.logaddexp(0.0, z)
        assert st == 0 and abs(y[0, 0] - want) <= 1e-9 * max(1.0, want), (z, y[0, 0], want)


def pin_lfilter(o, seed=5):
    """Scalar channel, constant step: the recurrence is the IIR filter
    h_t = dA h_{t-1} + (dt x~_t B_t), i.e. scipy.signal.lfilter([1], [1, -dA])."""
    from scipy.signal import lfilter
    rng = np.random.default_rng(seed)
    T, H, P, N, G, W = 12, 1, 1, 1, 1, 4
    u = rand_unit(rng, T, H, P, N, G, W)
    u["dt_raw"][:] = 0.3
    parent = np.arange(-1, T - 1, dtype=np.int32)
    y, st, _ = o.verify(parent, u, H, P, N, G, W)
    assert st == 0
    dt = np.logaddexp(0.0, 0.3 + u["dt_bias"][0])
    dA = np.exp(dt * u["A"][0])
    seq = np.concatenate([u["window"][:, 0], u["x"][:, 0]])
    xt = np.correlate(seq, u["conv_w"][0], mode="valid")
    drive = dt * xt * u["B"][:, 0, 0]
    h, _ = lfilter([1.0], [1.0, -dA], drive, zi=[dA * u["state"][0, 0, 0]])
    want = u["C"][:, 0, 0] * h + u["D"][0] * xt
    close(y[:, 0], want, 1e-12, "lfilter")


def pin_special_cases(o, seed=6):
    rng = np.random.default_rng(seed)
    H, P, N, G, W = 2, 2, 3, 1, 4
    T = 6
    parent = np.array([-1, 0, 0, 1, 1, 2], np.int32)
    # (i) step size -> 0: dA = 1 and no update, every node sees h0
    u = rand_unit(rng, T, H, P, N, G, W)
    u["dt_raw"][:] = -1e4
    y, _, _ = o.verify(parent, u, H, P, N, G, W)
    u0 = dict(u, C=np.zeros_like(u["C"]))
    yD, _, _ = o.verify(parent, u0, H, P, N, G, W)  # = D x~ only
    for v in range(T):
        for h in range(H):
            for p in range(P):
                c = h * P + p
                close(y[v, c] - yD[v, c], u["C"][v, 0] @ u["state"][h, p], 1e-12, "dt->0")
    # (ii) zero root state, one node: y = dt (C.B) x~ + D x~
    u = rand_unit(rng, 1, H, P, N, G, W)
    u["state"][:] = 0.0
    y, _, _ = o.verify(np.array([-1], np.int32), u, H, P, N, G, W)
    seq = np.concatenate([u["window"], u["x"]])
    for h in range(H):
        dt = np.logaddexp(0.0, u["dt_raw"][0, h] + u["dt_bias"][h])
        for p in range(P):
            c = h * P + p
            xt = float(np.dot(u["conv_w"][c], seq[:, c]))
            close(y[0, c], dt * float(u["C"][0, 0] @ u["B"][0, 0]) * xt + u["D"][h] * xt, 1e-12, "h0=0")
    # (iii) identity conv weights give x~ = x; W = 1 gives x~ = w x
    for Wc in (4, 1):
        u = rand_unit(rng, T, H, P, N, G, Wc)
        u["C"][:] = 0.0
        u["conv_w"][:] = 0.0
        u["conv_w"][:, Wc - 1] = 1.0 if Wc > 1 else 1.7
        y, _, _ = o.verify(parent, u, H, P, N, G, Wc)
        scale = 1.0 if Wc > 1 else 1.7
        want = u["x"] * scale * np.repeat(u["D"], P)[None, :]
        close(y, want, 1e-14, "identity conv W=%d" % Wc)
    # (iv) C = 0 and D = 0 give exactly zero
    u = rand_unit(rng, T, H, P, N, G, W)
    u["C"][:] = 0.0
    u["D"][:] = 0.0
    y, _, _ = o.verify(parent, u, H, P, N, G, W)
    assert np.all(y == 0.0)
    # (v) y is affine in h0
    u = rand_unit(rng, T, H, P, N, G, W)
    y1, _, _ = o.verify(parent, u, H, P, N, G, W)
    y2, _, _ = o.verify(parent, dict(u, state=2 * u["state"]), H, P, N, G, W)
    y0, _, _ = o.verify(parent, dict(u, state=0 * u["state"]), H, P, N, G, W)
    close(y2 - y0, 2 * (y1 - y0), 1e-12, "affine in h0")


def pin_commit(o, seed=7):
    rng = np.random.default_rng(seed)
    for (H, P, N, G, W, silu, cb, xbc, gate) in all_shapes():
        T = 9
        parent = _rand_parent(rng, T)
        u = rand_unit(rng, T + 1, H, P, N, G, W, conv_b=cb, xbc=xbc, gate=gate)
        uT = take(u, range(T))
        # length 0 is the identity, bit for bit
        so, wo, st = o.commit(parent, np.zeros(0, np.int32), 0, uT, H, P, N, G, W, silu, xbc)
        assert st == 0 and np.array_equal(so, uT["state"]) and np.array_equal(wo, uT["window"])
        # commit then a 1-node verify of the next token == scan over prefix + token
        leaf = int(rng.integers(T))
        pth = root_path(parent, leaf)
        so, wo, st = o.commit(parent, np.array(pth, np.int32), len(pth), uT, H, P, N, G, W, silu, xbc)
        assert st == 0
        nxt = dict(take(u, [T]), state=so, window=wo)
        y1, st1, _ = o.verify(np.array([-1], np.int32), nxt, H, P, N, G, W, silu, xbc)
        ys, hs, ws = o.scan(take(u, pth + [T]), len(pth) + 1, H, P, N, G, W, silu, xbc)
        close(y1[0], ys[-1], 1e-12, "commit then decode")
        so2, wo2, _ = o.commit(np.array([-1], np.int32), np.array([0], np.int32), 1, nxt, H, P, N, G, W, silu, xbc)
        close(so2, hs, 1e-12, "commit+commit state")
        assert np.array_equal(wo2, ws)
        # two commits along a split path == one commit of the whole path
        if len(pth) >= 2:
            k = len(pth) // 2
            a, _, _ = o.commit(parent, np.array(pth[:k], np.int32), k, uT, H, P, N, G, W, silu, xbc)
            sub = take(uT, pth[k:])
            sub_parent = np.arange(-1, len(pth) - k - 1, dtype=np.int32)
            sa, wa, _ = o.commit(parent, np.array(pth[:k], np.int32), k, uT, H, P, N, G, W, silu, xbc)
            sb, wb, _ = o.commit(sub_parent, np.arange(len(pth) - k, dtype=np.int32), len(pth) - k,
                                 dict(sub, state=sa, window=wa), H, P, N, G, W, silu, xbc)
            close(sb, so, 1e-12, "two commits == one")
            assert np.array_equal(wb, wo)
            del a
        # an invalid path leaves outputs untouched and reports E_PATH
        if len(pth) >= 1:
            bad = np.array(pth[::-1], np.int32) if len(pth) > 1 else np.array([T], np.int32)
            so3, wo3, st3 = o.commit(parent, bad, len(bad), uT, H, P, N, G, W, silu, xbc)
            assert st3 == -11 and np.array_equal(so3, uT["state"]) and np.array_equal(wo3, uT["window"])


def pin_sibling_relabel(o, seed=8):
    """Another valid BFS labelling of the same tree permutes y the same way."""
    rng = np.random.default_rng(seed)
    H, P, N, G, W = 2, 2, 3, 1, 3
    parent = np.array([-1, 0, 0, 0, 1, 1, 3, 3, 3], np.int32)
    T = len(parent)
    u = rand_unit(rng, T, H, P, N, G, W)
    y, _, _ = o.verify(parent, u, H, P, N, G, W)
    # swap subtrees of siblings 1 and 3 (and order their children accordingly)
    perm_old = [0, 3, 2, 1, 6, 7, 8, 4, 5]  # new label k holds old node perm_old[k]
    new_of = {old: k for k, old in enumerate(perm_old)}
    parent2 = np.array([-1 if parent[o_] < 0 else new_of[int(parent[o_])] for o_ in perm_old], np.int32)
    assert o.validate_tree(parent2) == 0, parent2
    u2 = dict(u)
    for k in ("x", "B", "C", "dt_raw"):
        u2[k] = u[k][perm_old]
    y2, _, _ = o.verify(parent2, u2, H, P, N, G, W)
    assert np.array_equal(y2, y[perm_old])


def _is_bfs_labelling(parent):
    """Independent definition: run a queue-based BFS from the root-level
    nodes, visiting children in index order; a valid labelling is one whose
    visit order is 0, 1, 2, ... and whose links point into range."""
    T = len(parent)
    if T == 0:
        return True
    if any(not (-1 <= int(p) < T) for p in parent):
        return False
    if any(int(parent[i]) == i for i in range(T)):
        return False
    kids = {i: [] for i in range(-1, T)}
    for i in range(T):
        kids[int(parent[i])].append(i)
    order, q, seen = [], [-1], set()
    while q:
        v = q.pop(0)
        for c in kids[v]:
            if c in seen:
                return False
            seen.add(c)
            order.append(c)
            q.append(c)
    return order == list(range(T))


def pin_validator(o, tmax=5):
    for T in range(0, tmax + 1):
        for parent in itertools.product(range(-2, T + 1), repeat=T):
            p = np.array(parent, np.int32)
            want = 0 if _is_bfs_labelling(p) else -10
            got = o.validate_tree(p)
            assert got == want, (parent, got, want)


def _is_root_path(parent, path):
    """Independent definition of an accepted path: its length is between 0
    and the node count, every entry names a node, and the entries are
    exactly the root path of the last entry, root-level node first."""
    T, n = len(parent), len(path)
    if n == 0:
        return True
    if n > T or any(not (0 <= int(v) < T) for v in path):
        return False
    return [int(v) for v in path] == root_path(parent, int(path[-1]))


def pin_path_validator(o, tmax=4, sample_t5=4000, seed=11):
    """Every path of length 0..T+1 over the alphabet -1..T, for every BFS
    forest of up to `tmax` nodes, classified like the independent
    definition; for 5-node forests every valid path plus a random sample of
    invalid ones (starts below the root, broken links, ids out of range,
    one entry too many)."""
    for T in range(0, tmax + 1):
        for parent in all_bfs_forests(T):
            for n in range(0, T + 2):
                for path in itertools.product(range(-1, T + 1), repeat=n):
                    q = np.array(path, np.int32)
                    want = 0 if _is_root_path(parent, q) else -11
                    got = o.validate_path(parent, q, n)
                    assert got == want, (parent.tolist(), path, got, want)
    rng = np.random.default_rng(seed)
    forests = list(all_bfs_forests(5))
    for parent in forests:
        for v in range(5):
            q = np.array(root_path(parent, v), np.int32)
            assert o.validate_path(parent, q, len(q)) == 0, (parent.tolist(), q.tolist())
            if len(q) >= 2:
                # the same path with its root-level node cut off starts below the root
                assert o.validate_path(parent, q[1:], len(q) - 1) == -11, (parent.tolist(), q[1:].tolist())
    for _ in range(sample_t5):
        parent = forests[int(rng.integers(len(forests)))]
        n = int(rng.integers(0, 7))
        q = rng.integers(-1, 6, size=n).astype(np.int32)
        want = 0 if _is_root_path(parent, q) else -11
        assert o.validate_path(parent, q, n) == want, (parent.tolist(), q.tolist())
    # an invalid tree is reported as such, whatever the path
    assert o.validate_path(np.array([0, 0], np.int32), np.zeros(0, np.int32), 0) == -10


def pin_plan(o, seed=9):
    rng = np.random.default_rng(seed)
    cases = [np.arange(-1, 12, dtype=np.int32), np.array([-1] + [0] * 11, np.int32),
             np.array([-1, -1, 0, 0, 1, 2, 2, 3], np.int32)]
    cases += [_rand_parent(rng, int(rng.integers(1, 20))) for _ in range(20)]
    for parent in cases:
        T = len(parent)
        for W in (1, 2, 3, 4):
            st, plan, info = o.plan(parent, W)
            assert st == 0
            kids = [[i for i in range(T) if parent[i] == v] for v in range(T)]
            internal = [v for v in range(T) if kids[v]]
            for v in range(T):
                pth = root_path(parent, v)
                assert plan[v, 0] == len(pth)
                assert plan[v, 1] == parent[v]
                assert plan[v, 2] == (kids[v][0] if kids[v] else -1)
                assert plan[v, 3] == len(kids[v])
                assert plan[v, 4] == (internal.index(v) if kids[v] else -1)
                # conv inputs: the path read backwards, then window rows newest first
                seq = [-(1 + r) for r in range(W - 1)] + pth  # window rows oldest first, then path
                for j in range(1, 4):
                    want = seq[len(seq) - 1 - j] if j < W else -32768
                    assert plan[v, 4 + j] == want, (parent.tolist(), W, v, j, plan[v].tolist())
            # FIFO simulation (queue of internal nodes)
            q, peak = [], 0
            q.extend([i for i in range(T) if parent[i] == -1 and kids[i]])
            peak = max(peak, len(q))
            while q:
                cur = q.pop(0)
                for c in kids[cur]:
                    if kids[c]:
                        q.append(c)
                        peak = max(peak, len(q))
            assert info["peak_fifo"] == peak, (parent.tolist(), info, peak)
            assert info["max_depth"] == max((len(root_path(parent, v)) for v in range(T)), default=0)
            assert info["n_internal"] == len(internal)


def pin_peak_from_verify(o):
    """The literal walk's queue peak equals the plan's FIFO occupancy."""
    rng = np.random.default_rng(10)
    H, P, N, G, W = 1, 1, 2, 1, 2
    for _ in range(15):
        T = int(rng.integers(1, 16))
        parent = _rand_parent(rng, T)
        u = rand_unit(rng, T, H, P, N, G, W)
        _, _, pk = o.verify(parent, u, H, P, N, G, W)
        _, _, info = o.plan(parent, W)
        assert pk == info["peak_fifo"], (parent.tolist(), pk, info)


def pin_golden(o):
    for name in sorted(os.listdir(GOLDEN)):
        if not name.startswith("hand_") or not name.endswith(".json"):
            continue
        with open(os.path.join(GOLDEN, name)) as f:
            g = json.load(f)
        dm = g["dims"]
        H, P, N, G, W = dm["H"], dm["P"], dm["N"], dm["G"], dm["W"]
        u = {k: (None if v is None else np.array(v, np.float64)) for k, v in g["inputs"].items()}
        parent = np.array(g["parent"], np.int32)
        y, st, _ = o.verify(parent, u, H, P, N, G, W)
        assert st == 0
        close(y.reshape(-1), np.array(g["expect"]["y"], np.float64).reshape(-1), 1e-13, name + " y")
        for cm in g["expect"]["commits"]:
            pth = np.array(cm["path"], np.int32)
            so, wo, cst = o.commit(parent, pth, len(pth), u, H, P, N, G, W)
            assert cst == 0
            close(so.reshape(-1), np.array(cm["state"]).reshape(-1), 1e-13, name + " commit state")
            assert np.array_equal(wo.reshape(-1), np.array(cm["window"], np.float64).reshape(-1))




def pin_option_special_cases(o, seed=8):
    """The Mamba2-convention options against exact special cases:
    (i) gate input z = 0 gives y = 0 exactly (silu(0) = 0);
    (ii) with xbc, identity taps on the B and C channels (weight 1 on the
    current token, no bias, no activation) give exactly the plain result,
    since the convolved B and C then equal the raw ones;
    (iii) a huge z makes the gate the identity times z up to e^-z terms."""
    rng = np.random.default_rng(seed)
    H, P, N, G, W = 2, 3, 4, 2, 4
    T = 7
    parent = np.array([-1, 0, 0, 1, 1, 2, 5], np.int32)
    d, gn = H * P, G * N
    u = rand_unit(rng, T, H, P, N, G, W, gate=True)
    u["z"][:] = 0.0
    y, st, _ = o.verify(parent, u, H, P, N, G, W)
    assert st == 0 and np.all(y == 0.0), "gate with z = 0"
    u = rand_unit(rng, T, H, P, N, G, W, xbc=True)
    u["conv_w"][d:] = 0.0
    u["conv_w"][d:, W - 1] = 1.0
    y_x, st, _ = o.verify(parent, u, H, P, N, G, W, False, True)
    plain = dict(u, window=np.ascontiguousarray(u["window"][:, :d]), conv_w=np.ascontiguousarray(u["conv_w"][:d]))
    y_p, _, _ = o.verify(parent, plain, H, P, N, G, W)
    assert st == 0 and np.array_equal(y_x, y_p), "xbc with identity B/C taps"
    u = rand_unit(rng, T, H, P, N, G, W, gate=True)
    y_g, _, _ = o.verify(parent, dict(u, z=np.full((T, d), 40.0)), H, P, N, G, W)
    y_n, _, _ = o.verify(parent, dict(u, z=None), H, P, N, G, W)
    close(y_g, 40.0 * y_n, 1e-15, "gate with z = 40")


def pin_round_bf16(o, seed=10):
    """bf16 storage rounding of a committed state against its definition:
    bf16 values stay put; exact ties go to the even significand (worked
    values in a normal binade, in the subnormal range and at the overflow
    edge); any other value goes to the nearer of its bf16 neighbours,
    enumerated from float32 bit patterns; the reported gap is the distance
    to the nearest midpoint between neighbours."""
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 1 << 16, 4000).astype(np.uint32)
    vals = (bits << 16).view(np.float32).astype(np.float64)
    vals = vals[np.isfinite(vals)]
    r, _ = o.round_bf16(vals)
    assert np.array_equal(r, vals), "a bf16 value moved"
    sub, top = 2.0 ** -133, 255.0 * 2.0 ** 120
    worked = [(1 + 2 ** -8, 1.0), (1 + 3 * 2 ** -8, 1 + 2 ** -6), (-(1 + 2 ** -8), -1.0),
              (1 + 2 ** -8 + 2 ** -30, 1 + 2 ** -7), (1 + 2 ** -8 - 2 ** -30, 1.0),
              (0.75 + 2 ** -10, 0.75), (0.75 + 3 * 2 ** -10, 0.75 + 2 ** -8),
              (0.5 * sub, 0.0), (1.5 * sub, 2 * sub), (2.5 * sub, 2 * sub), (-3.5 * sub, -4 * sub),
              (2.0 ** 127 * (1 + 2 ** -8), 2.0 ** 127), (top + 2.0 ** 119, np.inf),
              (top + 2.0 ** 119 - 2.0 ** 100, top), (-(top + 2.0 ** 119), -np.inf), (1e39, np.inf)]
    xs = np.array([w[0] for w in worked])
    r, _ = o.round_bf16(xs)
    for (x, want), got in zip(worked, r):
        assert got == want, "round_bf16(%r) = %r, want %r" % (x, got, want)
    # random magnitudes across the float32 range, both signs
    n = 20000
    x = np.ldexp(1.0 + rng.random(n), rng.integers(-140, 127, n)) * rng.choice([-1.0, 1.0], n)
    r, gap = o.round_bf16(x)
    f32 = x.astype(np.float32)
    hi16 = (f32.view(np.uint32) >> 16).astype(np.int64)
    cand = np.stack([hi16 + k for k in (-1, 0, 1, 2)], axis=1)
    cval = ((cand.astype(np.uint32) & 0xFFFF) << 16).view(np.float32).astype(np.float64)
    dist = np.abs(cval - x[:, None])
    dist[~np.isfinite(cval)] = np.inf  # patterns next to zero or infinity that are not values
    best = dist.min(axis=1)
    on_tie = (dist == best[:, None]).sum(axis=1) > 1
    pick = cval[np.arange(n), dist.argmin(axis=1)]
    even = cval[np.arange(n), np.argmax((dist == best[:, None]) & (cand % 2 == 0), axis=1)]
    want = np.where(on_tie, even, pick)
    assert np.array_equal(r, want), "not the nearest bf16 value"
    srt = np.sort(np.where(np.isfinite(cval), cval, np.nan), axis=1)
    mids = 0.5 * (srt[:, 1:] + srt[:, :-1])
    gap_want = np.nanmin(np.abs(mids - x[:, None]), axis=1) / np.abs(x)
    close(gap, gap_want, 1e-12, "distance to the nearest rounding boundary")


ALL_PINS = [pin_chain_is_scan, pin_every_node_is_its_path_scan, pin_bruteforce_forests, pin_closed_form,
            pin_softplus_library, pin_lfilter, pin_special_cases, pin_commit, pin_sibling_relabel,
            pin_validator, pin_path_validator, pin_plan, pin_peak_from_verify, pin_golden, pin_option_special_cases,
            pin_round_bf16]
