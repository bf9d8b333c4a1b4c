"""ssm_tree_commit_verify_noalloc against ssm_tree_commit_verify.

The allocation-free round runs the same kernels as ssm_tree_commit_verify;
only the xBC conv's workspace moves from a stream-ordered pool allocation to
the library's fixed device array.  Its outputs (state, window, y, both
status arrays) must equal the allocating entry point's bit for bit, on calls
in a row that reuse the array (the second smaller than the first, with the
array still holding the first call's rows), with and without the options;
a call that needs more than the array holds is refused before anything is
enqueued; and a round captured in a HIP graph replays to the eager results.  Both entry points are called through the C ABI (the binding's
ctypes functions).
"""
import os
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import mamba2_tree_verification_amd as m  # noqa: E402
from testgen import configs as C  # noqa: E402
from tests.gpu_util import log  # noqa: E402
from tests.test_gpu_commit_verify import Step  # noqa: E402

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 32 << 20  # the fixed array of the allocation-free entry point


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load()


def _run(step, noalloc):
    cfg, gp, gn = step.cfg, step.gp, step.gn
    s_out = torch.full_like(gp.state, -777.0)
    w_out = torch.zeros_like(gp.window)
    y = torch.full((cfg.L, cfg.Bsz, cfg.T, cfg.d_in), float("nan"), dtype=torch.float32, device="cuda")
    cst = torch.full((cfg.Bsz,), 12345, dtype=torch.int32, device="cuda")
    vst = torch.full((cfg.Bsz,), 12345, dtype=torch.int32, device="cuda")
    m.commit_verify(step.dims, step.prm, gp.parent, gp.path, gp.path_len, gp.x, gp.B, gp.dt_raw, gp.window,
                    gp.state, w_out, s_out, gn.parent, gn.x, gn.B, gn.C, gn.dt_raw, y, cst, vst,
                    C_prev=gp.C if cfg.xbc else None, z=gn.z, noalloc=noalloc)
    torch.cuda.synchronize()
    return s_out, w_out, y, cst, vst


def _workspace_bytes(cfg):
    return cfg.L * cfg.Bsz * cfg.G * (cfg.T * 3 * cfg.N + 256) * 4 if cfg.xbc and cfg.T <= 16 else 0


def _same(a, b, what):
    for name, u, v in zip(("state", "window", "y", "commit status", "verify status"), a, b):
        assert u.dtype == v.dtype and u.shape == v.shape, (what, name)
        # bit for bit: the same kernels on the same inputs (NaN rows of an
        # invalid tree compare by their bits too)
        assert torch.equal(u.view(torch.int32) if u.dtype == torch.float32 else u,
                           v.view(torch.int32) if v.dtype == torch.float32 else v), (what, name)


# T, H, P, N, G, W, bf16, silu, conv_b, xbc, gate; L and Bsz
CASES = [
    ((16, 4, 64, 128, 1, 4, True, True, True, True, True), 3, 6),   # the larger call first
    ((9, 2, 64, 64, 2, 3, True, False, False, True, False), 2, 3),  # then a smaller one
    ((12, 4, 32, 32, 1, 4, False, True, True, True, True), 2, 2),   # fp32 inputs
    ((16, 4, 64, 128, 1, 4, True, True, False, False, False), 2, 4),  # no options: no scratch used
    ((20, 4, 64, 128, 1, 4, True, True, False, True, True), 2, 3),  # options past 16 nodes: the two calls
    ((40, 8, 64, 128, 1, 4, True, True, False, False, False), 2, 2),  # the one-launch 17-64-node round
]


def test_noalloc_matches_the_allocating_round():
    for i, (spec, L, Bsz) in enumerate(CASES):
        T, H, P, N, G, W, bf16, silu, cb, xbc, gate = spec
        cfg = C.Config(880 + i, "noalloc", L, Bsz, T, H, P, N, G, W, bf16, 0.5, "forest", silu, cb, xbc, gate)
        assert _workspace_bytes(cfg) <= SCRATCH_BYTES
        log("noalloc round %d: %s L=%d Bsz=%d, %d scratch bytes" % (i, spec, L, Bsz, _workspace_bytes(cfg)))
        step = Step(cfg)
        ref = _run(step, noalloc=False)
        got = _run(step, noalloc=True)
        _same(ref, got, "case %d" % i)
        again = _run(step, noalloc=True)  # a second call over the array the first one left
        _same(ref, again, "case %d repeated" % i)


def test_noalloc_full_size_round():
    """The 2.7B batch-16 tree-16 round with SiLU, the xBC conv and the gate
    (26.2 MB of convolved rows in the 32 MiB array), then the small
    workload's round over the same array."""
    big = C.CONFIGS[3].replace(cid=890, silu=True, xbc=True, gate=True)
    small = C.CONFIGS[0].replace(cid=891, silu=True, xbc=True, gate=True)
    assert _workspace_bytes(small) < _workspace_bytes(big) <= SCRATCH_BYTES
    for cfg in (big, small):
        log("noalloc round %s" % cfg.name)
        step = Step(cfg)
        _same(_run(step, noalloc=False), _run(step, noalloc=True), cfg.name)


def test_noalloc_refuses_a_call_beyond_its_scratch():
    # 32 x 32 sequences of 16-node trees, d_state 256: 51.4 MB of convolved
    # rows, more than the array holds; refused before anything is enqueued
    L, Bsz, T, H, P, N, G, W = 32, 32, 16, 1, 64, 256, 1, 4
    cfg = C.Config(892, "noalloc-big", L, Bsz, T, H, P, N, G, W, True, 0.5, "forest", True, False, True, False)
    assert _workspace_bytes(cfg) > SCRATCH_BYTES
    dims = m.make_dims(L, Bsz, T, H, P, N, G, W, True, True, xbc=True)
    dev = dict(device="cuda")
    CH = H * P + 2 * G * N
    A = torch.full((L, H), -1.0, **dev)
    prm = m.make_params(A, torch.zeros_like(A), torch.zeros_like(A), torch.zeros((L, CH, W), **dev), None)
    parent = torch.full((Bsz, T), -1, dtype=torch.int32, **dev)
    path = torch.zeros((Bsz, T), dtype=torch.int32, **dev)
    plen = torch.zeros((Bsz,), dtype=torch.int32, **dev)
    tok = torch.zeros((L, Bsz, T, H * P), dtype=torch.bfloat16, **dev)
    bc = torch.zeros((L, Bsz, T, G, N), dtype=torch.bfloat16, **dev)
    dt = torch.zeros((L, Bsz, T, H), dtype=torch.bfloat16, **dev)
    win = torch.zeros((L, Bsz, W - 1, CH), dtype=torch.bfloat16, **dev)
    state = torch.full((L, Bsz, H * P, N), 3.0, **dev)
    y = torch.full((L, Bsz, T, H * P), 5.0, **dev)
    with pytest.raises(m.SsmTreeError) as e:
        m.commit_verify(dims, prm, parent, path, plen, tok, bc, dt, win, state, win, state, parent, tok, bc, bc, dt,
                        y, C_prev=bc, noalloc=True)
    assert e.value.code == m.E_SCRATCH
    torch.cuda.synchronize()
    assert bool((state == 3.0).all()) and bool((y == 5.0).all())  # nothing ran


def test_noalloc_graph_replay_with_options():
    """The allocation-free round with the options (its fixed array in use)
    captured in a HIP graph and replayed three times, with unrelated eager
    work between replays, equals three eager rounds of
    ssm_tree_commit_verify bit for bit after every replay."""
    cfg = C.Config(893, "noalloc-graph", 2, 3, 12, 4, 64, 128, 1, 4, True, 0.5, "forest", True, True, True, True)
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
    _run(step, noalloc=True)  # an eager call first: the array's address is looked up there, not under capture
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    gp, gn = step.gp, step.gn
    cst = torch.empty((cfg.Bsz,), dtype=torch.int32, device="cuda")
    vst = torch.empty_like(cst)
    log("noalloc round captured in a graph: %s" % cfg.name)
    with torch.cuda.graph(graph, stream=side):
        m.commit_verify(step.dims, step.prm, gp.parent, gp.path, gp.path_len, gp.x, gp.B, gp.dt_raw, win, st, win,
                        st, gn.parent, gn.x, gn.B, gn.C, gn.dt_raw, y, cst, vst, C_prev=gp.C, z=gn.z, noalloc=True)
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
