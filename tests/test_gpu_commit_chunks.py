"""ssm_tree_commit along paths that span several of the commit kernel's
16-node chunks, against the float64 oracle.

Chain trees take accepted paths of fixed lengths around the chunk edges
(0, 1, 15, 16, 17, 32, 33, 47 and the whole chain), so one call holds
empty, single-node, exact-multiple and ragged last chunks side by side.
The shapes cover every d_state the kernel is built for, conv widths 1-4
(taps that reach back across a chunk edge and into the old window), one
to four heads per 64-channel block and a headdim whose heads straddle
blocks, bf16 and fp32 inputs, the xBC conv, and a bfloat16 state.
"""
import numpy as np
import pytest
import torch

import mamba2_tree_verification_amd as m
import oracle
from testgen import configs as C
from tests.gpu_util import GpuCase, check_commit, log, window_f64
from tests.test_gpu_state_bf16 import check_state

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load()


LENGTHS = [0, 1, 15, 16, 17, 32, 33, 47]

# T, H, P, N, G, W, bf16, silu, conv_b, xbc, state_bf16
SPECS = [
    (64, 4, 16, 16, 1, 1, False, False, False, False, False),   # four heads per block, no taps before the token
    (50, 4, 32, 32, 2, 2, True, True, True, False, False),      # two heads per block, two groups
    (64, 2, 64, 64, 1, 3, True, False, False, False, False),
    (48, 2, 64, 256, 1, 4, True, True, False, False, False),    # d_state 256
    (47, 8, 40, 128, 1, 4, False, True, True, False, False),    # headdim 40: blocks straddle heads
    (64, 2, 64, 32, 1, 4, True, True, True, True, False),       # xBC conv
    (64, 2, 64, 128, 1, 4, True, False, False, False, True),    # bfloat16 state
]


def _case(spec, cid):
    T, H, P, N, G, W, bf16, silu, cb, xbc, sbf = spec
    lengths = [n for n in LENGTHS if n <= T] + [T]
    cfg = C.Config(cid, "commit-chunks", 2, len(lengths), T, H, P, N, G, W, bf16, 0.5, "chain", silu, cb, xbc, False,
                   state_bf16=sbf)
    inp = C.make_inputs(cfg)
    for b, n in enumerate(lengths):
        inp.path[b, :] = -1
        inp.path[b, :n] = np.arange(n, dtype=np.int32)
        inp.path_len[b] = n
    return cfg, GpuCase(cfg, inp)


@pytest.mark.parametrize("inplace", [False, True], ids=["out", "inplace"])
@pytest.mark.parametrize("spec", SPECS, ids=lambda s: "T%dH%dP%dN%dG%dW%d%s%s%s" % (
    s[:6] + ("bf" if s[6] else "f32", "xbc" if s[9] else "", "sbf16" if s[10] else "")))
def test_commit_across_chunks(spec, inplace):
    cfg, case = _case(spec, 230 + SPECS.index(spec))
    log("commit across chunks %s %s lengths %s" % (spec, "in place" if inplace else "out of place",
                                                  list(case.inp.path_len)))
    s_in = case.g.state.clone()
    w_in = None if case.g.window is None else case.g.window.clone()
    s_out, w_out, st = case.commit(inplace=inplace, state=s_in, window=w_in)
    units = [(l, b) for l in range(cfg.L) for b in range(cfg.Bsz)]
    if not cfg.state_bf16:
        check_commit(case, s_out, w_out, st, units)
        return
    o = oracle.get()
    ref = case.oracle_commit(units)
    stn = st.cpu().numpy()
    for (l, b), (sr, wr, rc) in ref.items():
        assert stn[b] == rc == 0
        check_state(s_out[l, b].double().cpu().numpy(), sr, o, "state l=%d b=%d" % (l, b))
        assert np.array_equal(window_f64(cfg, w_out, l, b), wr)
