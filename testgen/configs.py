"""The five synthetic workloads and their tree / accepted-path generators.

Shapes follow the Mamba2 layer sizes the SpecMamba page evaluates on
(Mamba2-370M draft, Mamba2-2.7B target; SpecMamba page, section 4.3) and the
tree parameters it recommends (branching 2-3, depth 4-5, 12-16 predicted
tokens; SpecMamba page, section 5.2).  Value distributions:

  x, B, C, dt_raw, conv window ~ N(0, 1)        (inputs, bf16 except tiny)
  dt_bias ~ U(-4, -2) per (layer, head)
  A = -exp(U(0, ln 16)) per (layer, head)
  D ~ N(0, 1) per (layer, head)
  root SSM state ~ N(0, 0.1), N(0, 1) for the stress workload
  conv weights ~ N(0, 0.5); no conv bias
  gate input z ~ N(0, 1) (only with the gate option)

With the xbc option (conv over x, B and C, the Mamba2 convention) the conv
window, weights and bias span d_in + 2 G N channels: x, then B, then C.

N(m, s) names the standard deviation s.  bf16 inputs are float32 draws
rounded to nearest even.  Every tensor is a counter-based stream (seed,
stream id), so the (layer, sequence) slice of any tensor can be redrawn
alone.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import (DIST_NEG_EXP_UNIFORM, DIST_NORMAL, DIST_UNIFORM, as_f64, fill)

SEED_BASE = 0x55D00000

# stream ids, one per tensor
S_X, S_B, S_C, S_DT, S_WIN, S_STATE, S_DTB, S_A, S_D, S_CONVW, S_CONVB, S_Z = range(1, 13)


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    L: int
    Bsz: int
    T: int
    H: int
    P: int
    N: int
    G: int
    W: int
    bf16: bool
    state_std: float
    tree: str
    silu: bool = False
    conv_bias: bool = False
    xbc: bool = False
    gate: bool = False
    state_bf16: bool = False  # root state stored as bfloat16 (drawn, then rounded like the inputs)

    @property
    def d_in(self) -> int:
        return self.H * self.P

    @property
    def conv_ch(self) -> int:
        """Channels of the causal conv: x, or x, B and C with xbc."""
        return self.H * self.P + (2 * self.G * self.N if self.xbc else 0)

    @property
    def seed(self) -> int:
        return SEED_BASE + self.cid

    @property
    def e(self) -> int:
        return 2 if self.bf16 else 4

    def replace(self, **kw) -> "Config":
        d = dict(self.__dict__)
        d.update(kw)
        return Config(**d)


CONFIGS = {
    0: Config(0, "tiny-chain8-f32", 1, 1, 8, 4, 16, 16, 1, 4, False, 0.1, "chain"),
    1: Config(1, "mamba2-370m-chain16", 48, 1, 16, 32, 64, 128, 1, 4, True, 0.1, "chain"),
    2: Config(2, "mamba2-2.7b-tree16", 64, 1, 16, 80, 64, 128, 1, 4, True, 0.1, "rand_b3_d4"),
    3: Config(3, "mamba2-2.7b-batch16-tree16", 64, 16, 16, 80, 64, 128, 1, 4, True, 0.1, "spine_b23_d45"),
    4: Config(4, "mamba2-2.7b-batch64-tree64-stress", 64, 64, 64, 80, 64, 128, 1, 4, True, 1.0, "stress"),
}


# ----------------------------------------------------------------------------
# trees
# ----------------------------------------------------------------------------

def bfs_relabel(parent_of: list[int]) -> np.ndarray:
    """Relabel a tree given as creation-order parent links into BFS order.

    Children are visited in creation order, so the result has parent[i] < i,
    parent[] non-decreasing and every sibling range contiguous.
    """
    n = len(parent_of)
    kids = [[] for _ in range(n)]
    roots = []
    for i, p in enumerate(parent_of):
        (roots if p < 0 else kids[p]).append(i)
    order, q = [], list(roots)
    while q:
        v = q.pop(0)
        order.append(v)
        q.extend(kids[v])
    new = {old: k for k, old in enumerate(order)}
    out = np.full(n, -1, dtype=np.int32)
    for old in order:
        p = parent_of[old]
        out[new[old]] = -1 if p < 0 else new[p]
    return out


def chain(T: int) -> np.ndarray:
    return np.arange(-1, T - 1, dtype=np.int32)


def star(T: int) -> np.ndarray:
    p = np.zeros(T, dtype=np.int32)
    if T:
        p[0] = -1
    return p


def random_tree(rng: np.random.Generator, T: int, b_max: int, d_max: int, spine: int = 0) -> np.ndarray:
    """Single-root random attachment under branching <= b_max, depth <= d_max.

    A spine of `spine` nodes (a chain from the root) forces the realised
    depth to be at least `spine`.  Depth counts nodes on the root path, so
    the root has depth 1.
    """
    if T == 0:
        return np.zeros(0, dtype=np.int32)
    par, dep, nk = [-1], [1], [0]
    for _ in range(1, min(spine, T)):
        p = len(par) - 1
        par.append(p)
        dep.append(dep[p] + 1)
        nk.append(0)
        nk[p] += 1
    while len(par) < T:
        cand = [i for i in range(len(par)) if dep[i] < d_max and nk[i] < b_max]
        if not cand:
            raise ValueError("tree bounds too tight for %d nodes" % T)
        p = cand[int(rng.integers(len(cand)))]
        par.append(p)
        dep.append(dep[p] + 1)
        nk.append(0)
        nk[p] += 1
    return bfs_relabel(par)


def depths(parent: np.ndarray) -> np.ndarray:
    d = np.zeros(len(parent), dtype=np.int32)
    for i, p in enumerate(parent):
        d[i] = 1 if p < 0 else d[p] + 1
    return d


def root_path(parent: np.ndarray, v: int) -> list[int]:
    out = []
    while v >= 0:
        out.append(int(v))
        v = int(parent[v])
    return out[::-1]


def min_depth_for(b: int, T: int) -> int:
    d, cap = 1, 1
    while cap < T:
        d += 1
        cap = cap * b + 1 if b > 1 else cap + 1
    return d


def make_trees(cfg: Config, rng: np.random.Generator):
    """Return parent [Bsz][T] int32 and the accepted paths (path [Bsz][T], len [Bsz])."""
    T, Bsz = cfg.T, cfg.Bsz
    parent = np.zeros((Bsz, T), dtype=np.int32)
    path = np.full((Bsz, T), -1, dtype=np.int32)
    plen = np.zeros(Bsz, dtype=np.int32)
    for b in range(Bsz):
        kind = cfg.tree
        if kind == "chain":
            par = chain(T)
            L = int(rng.integers(0, T + 1))
            pth = list(range(L))
        elif kind == "rand_b3_d4":
            par = random_tree(rng, T, 3, 4)
            dep = depths(par)
            has_kid = np.zeros(T, bool)
            has_kid[par[par >= 0]] = True
            leaves = [i for i in range(T) if not has_kid[i]]
            leaf = leaves[int(rng.integers(len(leaves)))]
            pth = root_path(par, leaf)
            del dep
        elif kind == "spine_b23_d45":
            bb = int(rng.integers(2, 4))
            dd = int(rng.integers(4, 6))
            if bb == 2 and dd == 4:  # 1+2+4+8 = 15 < 16 nodes: not realisable
                dd = 5
            par = random_tree(rng, T, bb, dd, spine=dd)
            pth = _random_depth_path(rng, par)
        elif kind == "stress":
            if b == 0:
                par = chain(T)
            elif b == 1:
                par = star(T)
            else:
                bb = int(rng.integers(2, 5))
                dmin = min_depth_for(bb, T)
                dd = int(rng.integers(dmin, 9))
                par = random_tree(rng, T, bb, dd, spine=dd)
            pth = _random_depth_path(rng, par)
        elif kind == "forest":
            par = random_forest(rng, T)
            pth = random_prefix_path(rng, par)
        elif kind == "chain_or_star":
            par = chain(T) if b % 2 == 0 else star(T)
            pth = random_prefix_path(rng, par)
        else:
            raise ValueError(kind)
        parent[b] = par
        plen[b] = len(pth)
        path[b, : len(pth)] = pth
    return parent, path, plen


def random_forest(rng: np.random.Generator, T: int) -> np.ndarray:
    """Random BFS labelling, possibly several root-level nodes: each parent is
    drawn between the previous node's parent and i - 1."""
    if T == 0:
        return np.zeros(0, dtype=np.int32)
    p = [-1]
    for i in range(1, T):
        p.append(int(rng.integers(p[-1], i)))
    return np.array(p, dtype=np.int32)


def random_prefix_path(rng, par):
    """A prefix of the root path of a uniformly random node (length 0 allowed)."""
    T = len(par)
    if T == 0:
        return []
    v = int(rng.integers(T))
    full = root_path(par, v)
    return full[: int(rng.integers(0, len(full) + 1))]


def _random_depth_path(rng, par):
    dep = depths(par)
    L = int(rng.integers(0, int(dep.max(initial=0)) + 1))
    if L == 0:
        return []
    cands = np.nonzero(dep == L)[0]
    v = int(cands[int(rng.integers(len(cands)))])
    return root_path(par, v)


# ----------------------------------------------------------------------------
# tensors
# ----------------------------------------------------------------------------

@dataclass
class Inputs:
    cfg: Config
    parent: np.ndarray
    path: np.ndarray
    path_len: np.ndarray
    x: np.ndarray          # [L][Bsz][T][d_in]   (uint16 bf16 bits or float32)
    B: np.ndarray          # [L][Bsz][T][G][N]
    C: np.ndarray          # [L][Bsz][T][G][N]
    dt_raw: np.ndarray     # [L][Bsz][T][H]
    window: np.ndarray     # [L][Bsz][W-1][d_in]
    state: np.ndarray      # [L][Bsz][H][P][N] float32 (uint16 bf16 bits with state_bf16)
    A: np.ndarray          # [L][H] float32
    D: np.ndarray
    dt_bias: np.ndarray
    conv_w: np.ndarray     # [L][d_in][W] float32
    conv_b: np.ndarray | None = None
    z: np.ndarray | None = None   # [L][Bsz][T][d_in] gate input (gate option only)
    extra: dict = field(default_factory=dict)


def tensor_shapes(cfg: Config) -> dict:
    L, Bsz, T, H, P, N, G, W, d = cfg.L, cfg.Bsz, cfg.T, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.d_in
    ch = cfg.conv_ch
    return dict(x=(L, Bsz, T, d), B=(L, Bsz, T, G, N), C=(L, Bsz, T, G, N), dt_raw=(L, Bsz, T, H),
                window=(L, Bsz, W - 1, ch), state=(L, Bsz, H, P, N), A=(L, H), D=(L, H), dt_bias=(L, H),
                conv_w=(L, ch, W), conv_b=(L, ch), z=(L, Bsz, T, d))


# (stream, dist, a, b, is_input_dtype)
def _specs(cfg: Config) -> dict:
    return dict(
        x=(S_X, DIST_NORMAL, 0.0, 1.0, True),
        B=(S_B, DIST_NORMAL, 0.0, 1.0, True),
        C=(S_C, DIST_NORMAL, 0.0, 1.0, True),
        dt_raw=(S_DT, DIST_NORMAL, 0.0, 1.0, True),
        window=(S_WIN, DIST_NORMAL, 0.0, 1.0, True),
        state=(S_STATE, DIST_NORMAL, 0.0, cfg.state_std, False),
        A=(S_A, DIST_NEG_EXP_UNIFORM, 0.0, math.log(16.0), False),
        D=(S_D, DIST_NORMAL, 0.0, 1.0, False),
        dt_bias=(S_DTB, DIST_UNIFORM, -4.0, -2.0, False),
        conv_w=(S_CONVW, DIST_NORMAL, 0.0, 0.5, False),
        conv_b=(S_CONVB, DIST_NORMAL, 0.0, 0.5, False),
        z=(S_Z, DIST_NORMAL, 0.0, 1.0, True),
    )


def stored_bf16(cfg: Config, name: str) -> bool:
    """Whether tensor `name` is stored as bfloat16 bits."""
    return (_specs(cfg)[name][4] and cfg.bf16) or (name == "state" and cfg.state_bf16)


def draw(cfg: Config, name: str, shape=None, offset: int = 0, nthreads=None) -> np.ndarray:
    stream, dist, a, b, is_in = _specs(cfg)[name]
    shp = tensor_shapes(cfg)[name] if shape is None else shape
    return fill(shp, cfg.seed, stream, dist, a, b, bf16=stored_bf16(cfg, name), offset=offset, nthreads=nthreads)


def make_inputs(cfg: Config, nthreads=None, skip=()) -> Inputs:
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    parent, path, plen = make_trees(cfg, rng)
    skip = set(skip) | (set() if cfg.conv_bias else {"conv_b"}) | (set() if cfg.gate else {"z"})
    t = {k: (None if k in skip else draw(cfg, k, nthreads=nthreads)) for k in tensor_shapes(cfg)}
    return Inputs(cfg=cfg, parent=parent, path=path, path_len=plen, **t)


def unit_offsets(cfg: Config, l: int, b: int) -> dict:
    """Flat element offset of the (layer l, sequence b) slice of each tensor."""
    L, Bsz, T, H, P, N, G, W, d = cfg.L, cfg.Bsz, cfg.T, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.d_in
    u = l * Bsz + b
    ch = cfg.conv_ch
    return dict(x=u * T * d, B=u * T * G * N, C=u * T * G * N, dt_raw=u * T * H, window=u * (W - 1) * ch,
                state=u * H * P * N, A=l * H, D=l * H, dt_bias=l * H, conv_w=l * ch * W, conv_b=l * ch,
                z=u * T * d)


def unit_shapes(cfg: Config) -> dict:
    T, H, P, N, G, W, d = cfg.T, cfg.H, cfg.P, cfg.N, cfg.G, cfg.W, cfg.d_in
    ch = cfg.conv_ch
    return dict(x=(T, d), B=(T, G, N), C=(T, G, N), dt_raw=(T, H), window=(W - 1, ch), state=(H, P, N),
                A=(H,), D=(H,), dt_bias=(H,), conv_w=(ch, W), conv_b=(ch,), z=(T, d))


def unit_f64(cfg: Config, l: int, b: int, inputs: Inputs | None = None) -> dict:
    """float64 copies of every tensor slice that unit (l, b) reads.

    Taken from `inputs` when given, else redrawn from the counter streams
    (bit-identical either way).
    """
    offs, shp = unit_offsets(cfg, l, b), unit_shapes(cfg)
    out = {"conv_b": None, "z": None}
    for k in shp:
        if (k == "conv_b" and not cfg.conv_bias) or (k == "z" and not cfg.gate):
            continue
        if inputs is not None:
            full = getattr(inputs, k)
            if k in ("A", "D", "dt_bias", "conv_w", "conv_b"):
                arr = full[l]
            else:
                arr = full[l, b]
        else:
            arr = draw(cfg, k, shape=shp[k], offset=offs[k], nthreads=1)
        out[k] = as_f64(arr, stored_bf16(cfg, k)).reshape(shp[k])
    return out
