"""The C ABI on the CPU: the library loads, exports every declared symbol,
and rejects bad arguments on the host before anything is enqueued.

Every call here fails a host-side check, so no kernel is ever launched
(fake device addresses are never dereferenced)."""
import ctypes
import os
import re

import pytest

import mamba2_tree_verification_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_tree.h")


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char\s*\*)\s*(ssm_tree_\w+)\s*\(", src, re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(["ssm_tree_verify", "ssm_tree_commit", "ssm_tree_commit_verify",
                                           "ssm_tree_commit_verify_noalloc", "ssm_tree_plan",
                                           "ssm_tree_status_string", "ssm_tree_abi_version"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(m.lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert m.ssm_tree_abi_version() == m.SSM_TREE_ABI_VERSION


def test_header_constants_match_binding():
    src = open(HEADER).read()
    consts = dict((k, int(v)) for k, v in re.findall(r"#define (SSM_TREE_\w+) \(?(-?\d+)\)?", src))
    assert consts["SSM_TREE_ABI_VERSION"] == m.SSM_TREE_ABI_VERSION
    assert consts["SSM_TREE_BF16"] == m.SSM_TREE_BF16 and consts["SSM_TREE_F32"] == m.SSM_TREE_F32
    for k, v in dict(OK=m.OK, E_NULL=m.E_NULL, E_ALIGN=m.E_ALIGN, E_DIMS=m.E_DIMS, E_DTYPE=m.E_DTYPE,
                     E_ALIAS=m.E_ALIAS, E_HIP=m.E_HIP, E_FLAGS=m.E_FLAGS, E_SCRATCH=m.E_SCRATCH, E_TREE=m.E_TREE,
                     E_PATH=m.E_PATH).items():
        assert consts["SSM_TREE_" + k] == v, k
    assert consts["SSM_TREE_PLAN_HEADER"] == m.PLAN_HEADER and consts["SSM_TREE_PLAN_STRIDE"] == m.PLAN_STRIDE
    assert consts["SSM_TREE_PLAN_UNUSED"] == m.PLAN_UNUSED
    assert consts["SSM_TREE_CONV_SILU"] == m.SSM_TREE_CONV_SILU
    assert consts["SSM_TREE_VERIFY_FIFO"] == m.SSM_TREE_VERIFY_FIFO
    assert consts["SSM_TREE_CONV_XBC"] == m.SSM_TREE_CONV_XBC
    assert consts["SSM_TREE_STATE_BF16"] == m.SSM_TREE_STATE_BF16


def test_status_strings():
    for code in (m.OK, m.E_NULL, m.E_ALIGN, m.E_DIMS, m.E_DTYPE, m.E_ALIAS, m.E_HIP, m.E_FLAGS, m.E_SCRATCH,
                 m.E_TREE, m.E_PATH):
        s = m.ssm_tree_status_string(code)
        assert s and s != "unknown status"
    assert m.ssm_tree_status_string(-999) == "unknown status"


# fake, 16-byte aligned, widely separated addresses (never dereferenced)
BASE = 0x7F0000000000
GAP = 1 << 36


def fake(i, off=0):
    return BASE + i * GAP + off


def good_dims(**kw):
    d = dict(L=2, Bsz=3, T=16, H=4, P=64, N=128, G=1, W=4, bf16=True)
    d.update(kw)
    return m.make_dims(d["L"], d["Bsz"], d["T"], d["H"], d["P"], d["N"], d["G"], d["W"], d["bf16"])


def good_params(**kw):
    p = m.Params(fake(20), fake(21), fake(22), fake(23), None)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def verify_args(**kw):
    a = dict(parent=fake(1), x=fake(2), B=fake(3), C=fake(4), dt_raw=fake(5), z=None, window=fake(6), state=fake(7),
             y=fake(8), status=fake(9))
    a.update(kw)
    return a


def call_verify(dims, params, **kw):
    a = verify_args(**kw)
    return m.ssm_tree_verify(dims, params, a["parent"], a["x"], a["B"], a["C"], a["dt_raw"], a["z"], a["window"],
                             a["state"], a["y"], a["status"], None)


@pytest.mark.parametrize("dkw,code", [
    (dict(T=65), m.E_DIMS), (dict(T=-1), m.E_DIMS), (dict(N=100), m.E_DIMS), (dict(N=512), m.E_DIMS),
    (dict(W=0), m.E_DIMS), (dict(W=5), m.E_DIMS), (dict(H=4, G=3), m.E_DIMS), (dict(H=3, P=16), m.E_DIMS),
    (dict(H=2, P=64, G=2, N=16), None), (dict(H=3, P=64, G=3), None), (dict(H=4, P=32, G=4), m.E_DIMS),
])
def test_dims_checks(dkw, code):
    if code is None:  # valid dims: exercise a different failure so nothing launches
        assert call_verify(good_dims(**dkw), good_params(), x=None) == m.E_NULL
    else:
        assert call_verify(good_dims(**dkw), good_params()) == code


def test_dtype_flags_null_align_alias():
    d = good_dims()
    d.in_dtype = 7
    assert call_verify(d, good_params()) == m.E_DTYPE
    d = good_dims()
    d.flags = 16  # the first unassigned bit
    assert call_verify(d, good_params()) == m.E_FLAGS
    assert m.load().ssm_tree_verify(None, None, *([None] * 11)) == m.E_NULL
    assert m.load().ssm_tree_verify(ctypes.byref(good_dims()), None, *([None] * 11)) == m.E_NULL
    assert call_verify(good_dims(), good_params(A=None)) == m.E_NULL
    for k in ("parent", "x", "B", "C", "dt_raw", "state", "y", "window"):
        assert call_verify(good_dims(), good_params(), **{k: None}) == m.E_NULL, k
    for k in ("parent", "x", "B", "C", "dt_raw", "state", "y", "window", "status"):
        assert call_verify(good_dims(), good_params(), **{k: fake(10 + len(k), 8)}) == m.E_ALIGN, k
    assert call_verify(good_dims(), good_params(D=fake(21, 4))) == m.E_ALIGN
    # y overlapping an input, partially or fully
    assert call_verify(good_dims(), good_params(), y=fake(2, 1024)) == m.E_ALIAS
    assert call_verify(good_dims(), good_params(), y=fake(7)) == m.E_ALIAS
    assert call_verify(good_dims(), good_params(), status=fake(8, 64)) == m.E_ALIAS


def call_commit(dims, params, **kw):
    a = dict(parent=fake(1), path=fake(11), plen=fake(12), x=fake(2), B=fake(3), C=fake(4), dt_raw=fake(5),
             win_in=fake(6), state_in=fake(7), win_out=fake(16), state_out=fake(17), status=fake(9))
    a.update(kw)
    return m.ssm_tree_commit(dims, params, a["parent"], a["path"], a["plen"], a["x"], a["B"], a["C"], a["dt_raw"],
                             a["win_in"], a["state_in"], a["win_out"], a["state_out"], a["status"], None)


def test_commit_host_checks():
    d, p = good_dims(), good_params()
    assert call_commit(d, p, plen=None) == m.E_NULL
    assert call_commit(d, p, win_out=None) == m.E_NULL
    assert call_commit(d, p, state_out=fake(7, 4096)) == m.E_ALIAS          # partial overlap with state_in
    assert call_commit(d, p, win_out=fake(6, 2048)) == m.E_ALIAS            # partial overlap with window_in
    assert call_commit(d, p, state_out=fake(2)) == m.E_ALIAS                # over x
    assert call_commit(d, p, win_out=fake(17, 4096)) == m.E_ALIAS           # window_out inside state_out
    assert call_commit(d, p, state_out=fake(17, 8)) == m.E_ALIGN
    assert call_commit(d, p, status=fake(17)) == m.E_ALIAS


def call_commit_verify(dims, params, **kw):
    a = dict(pparent=fake(1), path=fake(11), plen=fake(12), x_prev=fake(13), B_prev=fake(14), C_prev=fake(24),
             dt_prev=fake(15), win_in=fake(6), state_in=fake(7), win_out=fake(16), state_out=fake(17),
             parent=fake(18), x=fake(2), B=fake(3), C=fake(4), dt_raw=fake(5), z=None, y=fake(8), cst=fake(9),
             vst=fake(19))
    noalloc = kw.pop("noalloc", False)
    a.update(kw)
    fn = m.ssm_tree_commit_verify_noalloc if noalloc else m.ssm_tree_commit_verify
    return fn(dims, params, a["pparent"], a["path"], a["plen"], a["x_prev"], a["B_prev"], a["C_prev"], a["dt_prev"],
              a["win_in"], a["state_in"], a["win_out"], a["state_out"], a["parent"], a["x"], a["B"], a["C"],
              a["dt_raw"], a["z"], a["y"], a["cst"], a["vst"], None)


@pytest.mark.parametrize("noalloc", [False, True], ids=["alloc", "noalloc"])
@pytest.mark.parametrize("dkw", [dict(), dict(T=40), dict(H=8, P=40, N=16)])
def test_commit_verify_host_checks(dkw, noalloc):
    """(ssm_tree_commit_verify_noalloc makes the same checks)"""
    # the same checks whichever way the call would run (fused kernel, or the two calls)
    d, p = good_dims(**dkw), good_params()
    for k in ("pparent", "path", "plen", "x_prev", "B_prev", "dt_prev", "state_in", "state_out", "parent", "x",
              "B", "C", "dt_raw", "y", "win_in", "win_out"):
        assert call_commit_verify(d, p, **{k: None}, noalloc=noalloc) == m.E_NULL, k
    for k in ("pparent", "x_prev", "state_out", "C", "y", "cst", "vst", "win_out"):
        assert call_commit_verify(d, p, **{k: fake(30, 8)}, noalloc=noalloc) == m.E_ALIGN, k
    assert call_commit_verify(d, p, state_out=fake(7, 4096), noalloc=noalloc) == m.E_ALIAS      # partial overlap with state_in
    assert call_commit_verify(d, p, win_out=fake(6, 2048), noalloc=noalloc) == m.E_ALIAS        # partial overlap with window_in
    assert call_commit_verify(d, p, y=fake(7), noalloc=noalloc) == m.E_ALIAS                    # y over state_in
    assert call_commit_verify(d, p, y=fake(6), noalloc=noalloc) == m.E_ALIAS                    # y over window_in
    assert call_commit_verify(d, p, y=fake(17), noalloc=noalloc) == m.E_ALIAS                   # y over state_out
    assert call_commit_verify(d, p, state_out=fake(13), noalloc=noalloc) == m.E_ALIAS           # over x_prev
    assert call_commit_verify(d, p, win_out=fake(4), noalloc=noalloc) == m.E_ALIAS              # over C
    assert call_commit_verify(d, p, cst=fake(19), noalloc=noalloc) == m.E_ALIAS                 # the two status arrays
    assert call_commit_verify(d, p, vst=fake(1), noalloc=noalloc) == m.E_ALIAS                  # status over parent_prev
    assert call_commit_verify(d, good_params(A=None), noalloc=noalloc) == m.E_NULL
    bad = good_dims(**dkw)
    bad.flags = 16  # the first unassigned bit
    assert call_commit_verify(bad, p, noalloc=noalloc) == m.E_FLAGS


def test_plan_host_checks():
    d = good_dims(T=70)
    assert m.ssm_tree_plan(d, fake(1), fake(2), None) == m.E_DIMS
    assert m.ssm_tree_plan(good_dims(), None, fake(2), None) == m.E_NULL
    assert m.ssm_tree_plan(good_dims(), fake(1, 4), fake(2), None) == m.E_ALIGN
    assert m.ssm_tree_plan(good_dims(), fake(1), fake(1, 64), None) == m.E_ALIAS


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    t = torch.zeros(4)
    with pytest.raises(ValueError):
        m.make_params(t, t, t, t)


def test_option_host_checks():
    """The xBC conv and the gate: null, alignment and alias checks on their
    arguments, and refusal of shapes no kernel takes (nothing launches)."""
    p = good_params()
    dx = good_dims()
    dx.flags = m.SSM_TREE_CONV_XBC
    # verify: the gate input is checked like any input
    assert call_verify(good_dims(), p, z=fake(30, 8)) == m.E_ALIGN
    assert call_verify(good_dims(), p, z=fake(8)) == m.E_ALIAS           # z over y
    assert call_verify(good_dims(), p, z=fake(30), status=fake(30, 64)) == m.E_ALIAS
    # shapes no kernel takes with an option: headdim not a multiple of 16,
    # fp32 inputs with 64 nodes and d_state 128 (LDS), the FIFO walk
    assert call_verify(good_dims(T=64, bf16=False), p, z=fake(30)) == m.E_DIMS
    assert call_verify(good_dims(H=8, P=40), p, z=fake(30)) == m.E_DIMS
    d = good_dims(T=64, bf16=False)
    d.flags = m.SSM_TREE_CONV_XBC
    assert call_verify(d, p) == m.E_DIMS
    d = good_dims()
    d.flags = m.SSM_TREE_VERIFY_FIFO
    assert call_verify(d, p, z=fake(30)) == m.E_DIMS
    # commit with xBC: C is required and checked; the window spans d_in + 2GN channels
    assert call_commit(dx, p, C=None) == m.E_NULL
    assert call_commit(dx, p, C=fake(4, 8)) == m.E_ALIGN
    assert call_commit(dx, p, C=fake(17)) == m.E_ALIAS                    # C under state_out
    # without xBC, C is ignored (may be NULL or anything)
    assert call_commit(good_dims(), p, C=None, plen=None) == m.E_NULL     # fails on path_len, not C
    # 2 layers x 3 sequences x 3 rows x (256 + 256) channels x 2 bytes = 18432 bytes: a window_out starting
    # 10000 bytes into window_in (past the 9216 bytes of x-only rows) overlaps it with rows d_in + 2GN wide
    assert call_commit(dx, p, win_out=fake(6, 10000)) == m.E_ALIAS
    # the fused round
    assert call_commit_verify(dx, p, C_prev=None) == m.E_NULL
    assert call_commit_verify(good_dims(), p, z=fake(8)) == m.E_ALIAS    # z over y
    assert call_commit_verify(good_dims(), p, z=fake(30, 8)) == m.E_ALIGN
    assert call_commit_verify(good_dims(T=64, bf16=False), p, z=fake(30)) == m.E_DIMS
    d = good_dims(T=64, bf16=False)
    d.flags = m.SSM_TREE_CONV_XBC
    assert call_commit_verify(d, p) == m.E_DIMS


def test_state_bf16_host_checks():
    """A bfloat16 root state: refused, before anything is enqueued, where no
    kernel takes it (the FIFO walk, the options, the vector-ALU shapes, fp32
    inputs with d_state 256 past 16 nodes), and its byte size is what the
    range checks use.  Every call here fails on a host check."""
    p = good_params()

    def sb(flags=0, **kw):
        d = good_dims(**kw)
        d.flags = m.SSM_TREE_STATE_BF16 | flags
        return d

    assert call_verify(sb(m.SSM_TREE_VERIFY_FIFO), p) == m.E_DIMS
    assert call_verify(sb(m.SSM_TREE_CONV_XBC), p) == m.E_DIMS
    assert call_verify(sb(), p, z=fake(30)) == m.E_DIMS                        # the gate
    assert call_verify(sb(H=8, P=40), p) == m.E_DIMS                          # headdim not a multiple of 16
    assert call_verify(sb(T=40, H=6, P=32, G=2), p) == m.E_DIMS               # 96-channel B/C groups, T > 16
    assert call_verify(sb(T=64, N=256, bf16=False), p) == m.E_DIMS            # fp32 in, N 256: 184 KiB of LDS
    assert call_commit_verify(sb(m.SSM_TREE_VERIFY_FIFO), p) == m.E_DIMS
    assert call_commit_verify(sb(T=20, H=8, P=40), p) == m.E_DIMS
    assert call_commit_verify(sb(), p, z=fake(30)) == m.E_DIMS
    # the state is 2 bytes per element with the flag: 2 x 3 x 256 x 128 x 2 = 393216 bytes, so
    # state_out 393200 bytes into state_in overlaps it; without the flag (4 bytes per element)
    # so does one 600000 bytes in (alias checks are the last before a launch, so only overlaps
    # are asserted here)
    assert call_commit(sb(), p, state_out=fake(7, 393200)) == m.E_ALIAS
    assert call_commit_verify(sb(), p, state_out=fake(7, 393200)) == m.E_ALIAS
    assert call_commit(good_dims(), p, state_out=fake(7, 600000)) == m.E_ALIAS


def test_noalloc_refuses_a_call_beyond_its_scratch_before_any_hip_call():
    """ssm_tree_commit_verify_noalloc: 32 x 32 sequences of 16-node trees at
    d_state 256 with the xBC conv need 51.4 MB of convolved rows, more than
    its 32 MiB array; the call is refused after the argument checks and
    before any HIP call (so it runs here without a GPU)."""
    d = good_dims(L=32, Bsz=32, T=16, H=1, P=64, N=256)
    d.flags |= m.SSM_TREE_CONV_XBC
    assert call_commit_verify(d, good_params(), noalloc=True) == m.E_SCRATCH
    # the argument checks still come first
    assert call_commit_verify(d, good_params(), noalloc=True, y=None) == m.E_NULL
